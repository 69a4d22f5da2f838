"""GPU parity of each libkalm entry point against the CPU oracle.

Every case feeds the same seeded synthetic inputs (encoder_decoder_document_amd.synth)
to the HIP path through the C ABI and to the fp64 oracle, then compares
element by element: integer outputs bit-exact, floating outputs within
|g - r| <= 2e-2 + 1e-2 |r| (bf16 storage, fp32 accumulation) or 1e-4 + 1e-4 |r|
(the fp32 path).  Sizes span several tiles and a ragged tail.
"""
import math
import sys
import zlib

import numpy as np
import pytest
import torch

import oracle
from encoder_decoder_document_amd import ops, synth
from parity_util import BF16_TOL, F32_TOL, assert_close, to_dev, to_np

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


# ------------------------------------------------------------------ a0 layout
@pytest.mark.parametrize("lq,D", [([16], 8), ([3, 1, 4, 1, 5], 7), ([64] * 3 + [512, 1, 77], 100),
                                  # more than one 1024-query scan step, and one query with many passages
                                  pytest.param([int(x) for x in synth.integers(17, 1, 600, 2500)], 3, id="q2500-d3"),
                                  pytest.param([300], 5000, id="q1-d5000")])
def test_pair_layout_bit_exact(lq, D):
    _announce(f"pair_layout queries={len(lq)} D={D}")
    lq = np.asarray(lq, np.int32)
    rows = int(D * lq.sum())
    got = ops.kalm_pair_layout(to_dev(lq, torch.int32), D, rows=rows)
    torch.cuda.synchronize()
    ref = oracle.pair_layout(lq, D)
    for k in ("cu_q", "doc_of_pair", "final_row", "h0_row", "h0_final", "cu_u"):
        assert np.array_equal(got[k].cpu().numpy(), ref[k]), k


def test_pair_layout_overflow_marks_pairs_invalid():
    # row offsets past INT32_MAX never wrap: such pairs get -1 offsets (the
    # attention skips them, the readout gives NaN); the rest are exact
    _announce("pair_layout int32 overflow")
    lq = np.array([1 << 29, (1 << 29) - 3, 5], np.int32)
    D = 3
    got = ops.kalm_pair_layout(to_dev(lq, torch.int32), D, with_h0_row=False)
    torch.cuda.synchronize()
    lim = (1 << 31) - 1
    start = np.concatenate([[0], np.cumsum(lq.astype(np.int64))])
    cu, fin, h0f = [], [], []
    for q in range(len(lq)):
        for d in range(D):
            r0 = D * int(start[q]) + d * int(lq[q])
            ok = r0 + int(lq[q]) <= lim
            cu.append(r0 if ok else -1)
            fin.append(r0 + int(lq[q]) - 1 if ok else -1)
            h0f.append(int(start[q]) + int(lq[q]) - 1 if ok else -1)
    total = D * int(start[-1])
    cu.append(total if total <= lim else -1)
    assert -1 in cu and cu[0] == 0
    assert got["cu_q"].cpu().tolist() == cu
    assert got["final_row"].cpu().tolist() == fin
    assert got["h0_final"].cpu().tolist() == h0f
    assert got["doc_of_pair"].cpu().tolist() == [p % D for p in range(len(lq) * D)]
    assert got["cu_u"].cpu().tolist() == [int(v) for v in start]


# ------------------------------------------------------------------ a1 pooling
def _pool_case(seed, D, T, H, chunk, bf16, general_mask=False, lens=None):
    x = synth.normal(seed, (D, T, H), 1.0, bf16)
    if general_mask:
        mask = synth.bernoulli_mask(seed + 1, 0.55, (D, T))
        mask[0] = 0
    else:
        if lens is None:
            lens = synth.integers(seed + 1, 0, T, D)
        lens = np.asarray(lens)
        mask = (np.arange(T)[None] < lens[:, None]).astype(np.uint8)
    x[mask == 0] = np.nan  # padding must never be read
    return x, mask


@pytest.mark.parametrize("D,T,H,chunk,bf16,general", [
    (13, 103, 640, 4, True, False),
    (9, 1024, 1152, 4, True, False),
    (8, 64, 64, 4, False, False),
    (11, 97, 640, 1, True, True),
    (7, 50, 256, 3, True, True),
    (6, 200, 128, 8, False, True),
    (5, 130, 640, 64, True, True),
])
def test_chunk_pool_parity(D, T, H, chunk, bf16, general):
    _announce(f"chunk_pool D={D} T={T} H={H} chunk={chunk} bf16={bf16} general={general}")
    lens = None
    if not general:
        lens = synth.integers(7 + D, 0, T, D)
        lens[:4] = [0, 1, min(T, 5), T]
    x, mask = _pool_case(100 + D, D, T, H, chunk, bf16, general, lens)
    dt = torch.bfloat16 if bf16 else torch.float32
    pooled, cm, nc = ops.kalm_chunk_pool(to_dev(x, dt), to_dev(mask, torch.uint8), chunk)
    torch.cuda.synchronize()
    rp, rcm, rnc = oracle.chunk_pool(x, mask, chunk)
    assert np.array_equal(cm.cpu().numpy(), rcm)
    assert np.array_equal(nc.cpu().numpy(), rnc)
    atol, rtol = BF16_TOL if bf16 else F32_TOL
    assert_close(to_np(pooled), rp, atol, rtol, "pooled")
    g = to_np(pooled)
    assert not g[rcm == 0].any(), "empty chunks must be written as 0"


def test_chunk_pool_constant_chunks_bit_exact():
    _announce("chunk_pool constant chunks")
    D, T, H = 6, 61, 640
    const = synth.normal(5, (D, -(-T // 4), H), 1.0, True)
    x = np.repeat(const, 4, axis=1)[:, :T].copy()
    lens = np.array([61, 60, 59, 1, 0, 33], np.int32)
    mask = (np.arange(T)[None] < lens[:, None]).astype(np.uint8)
    x[mask == 0] = np.nan
    pooled, cm, _ = ops.kalm_chunk_pool(to_dev(x, torch.bfloat16), to_dev(mask, torch.uint8), 4)
    torch.cuda.synchronize()
    g = pooled.float().cpu().numpy()
    c = cm.cpu().numpy() == 1
    assert np.array_equal(g[c], const[c])


# ------------------------------------------------------------------ a2 cross K/V
@pytest.mark.parametrize("D,C,H,kv,bf16", [(7, 37, 640, 256, True), (3, 256, 1152, 256, True),
                                           (2, 256, 2560, 1024, True), (5, 29, 640, 72, True),
                                           (8, 16, 64, 32, False)])
def test_cross_kv_parity(D, C, H, kv, bf16):
    _announce(f"cross_kv D={D} C={C} H={H} kv={kv} bf16={bf16}")
    pooled = synth.normal(20 + D, (D, C, H), 1.0, bf16)
    cm = synth.bernoulli_mask(21 + D, 0.7, (D, C))
    cm[0] = 0
    W = synth.normal(22 + D, (2 * kv, H), 0.02, bf16)
    dt = torch.bfloat16 if bf16 else torch.float32
    got = to_np(ops.kalm_cross_kv(to_dev(pooled, dt), to_dev(cm, torch.uint8), to_dev(W, dt)))
    torch.cuda.synchronize()
    K, V = oracle.cross_kv(pooled, W[:kv], W[kv:])
    ref = np.concatenate([K, V], -1) * (cm[..., None] != 0)
    atol, rtol = BF16_TOL if bf16 else F32_TOL
    assert_close(got, ref, atol, rtol, "KVc")
    assert not got[cm == 0].any()


def test_cross_kv_masked_rows_zero_on_the_big_tile_path():
    # >= 512 tiles of 256 x 256 (D = 100 passages of 256 chunks, 2 kv = 2048):
    # rows whose chunk mask is 0 are exactly 0 even though the pooled rows
    # behind them hold non-zero values; the valid rows match the oracle
    _announce("cross_kv masked, big-tile shape")
    D, C, H, kv = 100, 256, 640, 1024
    pooled = synth.normal(90, (D, C, H), 1.0, True)          # padded rows non-zero on purpose
    n_valid = synth.integers(91, 0, C, D)
    n_valid[:3] = [0, 128, 256]
    cm = (np.arange(C)[None] < n_valid[:, None]).astype(np.uint8)
    cm[5, ::3] = 0                                            # a general mask in one passage
    W = synth.normal(92, (2 * kv, H), 0.02, True)
    got = to_np(ops.kalm_cross_kv(to_dev(pooled, torch.bfloat16), to_dev(cm, torch.uint8),
                                  to_dev(W, torch.bfloat16)))
    torch.cuda.synchronize()
    assert not got[cm == 0].any(), "masked chunk rows must be written as 0"
    valid = cm != 0
    K, V = oracle.cross_kv(pooled[valid], W[:kv], W[kv:])
    assert_close(got[valid], np.concatenate([K, V], -1), *BF16_TOL, "KVc valid rows")


@pytest.mark.parametrize("D,C,H,kv,L,bf16", [(7, 37, 640, 256, 3, True), (50, 256, 1152, 256, 6, True),
                                             (8, 16, 64, 32, 2, False)])
def test_cross_kv_layers_parity(D, C, H, kv, L, bf16):
    # every layer's cross K/V in one launch equals each layer's projection
    # (layer l at columns [l 2kv, (l+1) 2kv) of every output row); masked rows 0
    _announce(f"cross_kv_layers D={D} C={C} H={H} kv={kv} L={L} bf16={bf16}")
    pooled = synth.normal(93 + D, (D, C, H), 1.0, bf16)
    cm = synth.bernoulli_mask(94 + D, 0.6, (D, C))
    cm[0] = 0
    W = synth.normal(95 + D, (L, 2 * kv, H), 0.02, bf16)
    dt = torch.bfloat16 if bf16 else torch.float32
    got = to_np(ops.kalm_cross_kv_layers(to_dev(pooled, dt), to_dev(cm, torch.uint8), to_dev(W, dt)))
    torch.cuda.synchronize()
    assert got.shape == (D, C, L, 2 * kv)
    assert not got[cm == 0].any()
    valid = cm != 0
    atol, rtol = BF16_TOL if bf16 else F32_TOL
    for l in range(L):
        K, V = oracle.cross_kv(pooled[valid], W[l, :kv], W[l, kv:])
        assert_close(got[valid][:, l], np.concatenate([K, V], -1), atol, rtol, f"KVc layer {l}")


# ------------------------------------------------------------------ a5 linear
@pytest.mark.parametrize("M,K,N,mode", [(1000, 1152, 1536, "bf16"), (300, 1024, 1152, "acc"),
                                        (77, 200, 136, "f32out"), (513, 640, 1536, "bf16"),
                                        (130, 64, 96, "f32"), (33, 36, 20, "f32acc"),
                                        # large enough for the big-tile paths (>= 512 tiles of 256 x 256),
                                        # ragged in M, and a K that is not a multiple of 64
                                        (22093, 1152, 1536, "bf16"), (22093, 1024, 1152, "acc"), (40003, 1024, 1152, "acc"),
                                        (88001, 1000, 1536, "bf16"),
                                        # the residual update's big-tile path with a ragged last column tile
                                        (40003, 1024, 1160, "acc"),
                                        # its split ring (activation copies a k-tile ahead): a K tail, and
                                        # k-loops of one and of two k-tiles
                                        (22093, 1000, 1536, "acc"), (22093, 64, 1536, "acc"), (22093, 128, 1536, "acc"),
                                        # a long k-loop: the residual update on the persistent 256 x 256 tiles,
                                        # ragged in M, and in N
                                        (22093, 2048, 1536, "acc"), (26200, 2048, 1160, "acc")])
def test_linear_parity(M, K, N, mode):
    _announce(f"linear M={M} K={K} N={N} mode={mode}")
    bf = mode in ("bf16", "acc", "f32out")
    X = synth.normal(30 + M, (M, K), 1.0, bf)
    W = synth.normal(31 + M, (N, K), 0.02, bf)
    dt = torch.bfloat16 if bf else torch.float32
    ref = X.astype(np.float64) @ W.astype(np.float64).T
    if mode == "bf16":
        got = to_np(ops.kalm_linear(to_dev(X, dt), to_dev(W, dt)))
        assert_close(got, ref, *BF16_TOL, "Y bf16")
    elif mode in ("acc", "f32acc"):
        Y0 = synth.normal(32 + M, (M, N), 1.0, False)
        Y = to_dev(Y0, torch.float32)
        Yb = torch.empty(M, N, dtype=torch.bfloat16, device="cuda") if mode == "acc" else None
        ops.kalm_linear(to_dev(X, dt), to_dev(W, dt), Y=Y, accumulate=True, Y_bf16=Yb)
        torch.cuda.synchronize()
        tol = (1e-4, 1e-4) if mode == "f32acc" else (1e-3, 1e-4)
        assert_close(to_np(Y), Y0 + ref, *tol, "Y += XW^T")
        if Yb is not None:
            assert torch.equal(Yb.cpu(), Y.cpu().to(torch.bfloat16)), "bf16 copy is RNE of the fp32 result"
    elif mode == "f32out":
        got = to_np(ops.kalm_linear(to_dev(X, dt), to_dev(W, dt), y_dtype=torch.float32))
        assert_close(got, ref, 1e-3, 1e-4, "Y f32")
    else:
        got = to_np(ops.kalm_linear(to_dev(X, dt), to_dev(W, dt)))
        assert_close(got, ref, *F32_TOL, "Y f32 path")


@pytest.mark.parametrize("M,K,N,bf,indexed", [(300, 1024, 1152, True, True), (40003, 1024, 1152, True, True),
                                               (40003, 1024, 1160, True, True),
                                               (22093, 1024, 1152, True, False), (33, 36, 20, False, True),
                                               # the gathered big-tile path with a K tail
                                               (22093, 1000, 1536, True, True)])
def test_linear_residual_parity(M, K, N, bf, indexed):
    """Y = R[r_row] + X W^T: the residual update starting from gathered rows
    (big and small tile paths, fp32 path); out-of-range indices give NaN rows."""
    _announce(f"linear_residual M={M} K={K} N={N} bf16={bf} indexed={indexed}")
    X = synth.normal(40 + M, (M, K), 1.0, bf)
    W = synth.normal(41 + M, (N, K), 0.02, bf)
    dt = torch.bfloat16 if bf else torch.float32
    rows = 97 if indexed else M
    R = synth.normal(42 + M, (rows, N), 1.0, False)
    idx = synth.integers(43 + M, 0, rows - 1, M) if indexed else None
    if indexed:
        idx[[1, M // 2]] = [rows, -1]  # out of range: NaN rows
    Yb = torch.empty(M, N, dtype=torch.bfloat16, device="cuda") if bf else None
    Y = ops.kalm_linear_residual(to_dev(X, dt), to_dev(W, dt), to_dev(R, torch.float32),
                                 to_dev(idx, torch.int32) if indexed else None, Y_bf16=Yb)
    torch.cuda.synchronize()
    ref = X.astype(np.float64) @ W.astype(np.float64).T
    base = R[np.clip(idx, 0, rows - 1)] if indexed else R
    ref = ref + base
    got = to_np(Y)
    if indexed:
        bad = np.zeros(M, bool)
        bad[[1, M // 2]] = True
        assert np.isnan(got[bad]).all()
        got, ref = got[~bad], ref[~bad]
    assert_close(got, ref, *((1e-3, 1e-4) if bf else (1e-4, 1e-4)), "Y = R[idx] + XW^T")
    if Yb is not None:  # NaN rows included
        assert np.array_equal(to_np(Yb), to_np(Y.to(torch.bfloat16)), equal_nan=True), \
            "bf16 copy is RNE of the fp32 result"


# ------------------------------------------------------------------ a3 merged attention
def _attn_case(seed, lqs, docs_c, Cmax, nq, nkv, d, bf16, std=0.7, general=False):
    P = len(lqs)
    D = len(docs_c)
    rows = int(sum(lqs))
    Q = synth.normal(seed, (rows, nq * d), std, bf16)
    Ks = synth.normal(seed + 1, (rows, nkv * d), std, bf16)
    Vs = synth.normal(seed + 2, (rows, nkv * d), 1.0, bf16)
    Kc = synth.normal(seed + 3, (D * Cmax, nkv * d), std, bf16)
    Vc = synth.normal(seed + 4, (D * Cmax, nkv * d), 1.0, bf16)
    if general:
        cm = synth.bernoulli_mask(seed + 5, 0.5, (D, Cmax))
    else:
        cm = (np.arange(Cmax)[None] < np.asarray(docs_c)[:, None]).astype(np.uint8)
    # masked chunks hold NaN: they must never be read
    Kc.reshape(D, Cmax, -1)[cm == 0] = np.nan
    Vc.reshape(D, Cmax, -1)[cm == 0] = np.nan
    doc_of_pair = (np.arange(P) % D).astype(np.int32)
    cu_q = np.concatenate([[0], np.cumsum(lqs)]).astype(np.int32)
    return Q, Ks, Vs, Kc, Vc, cm, doc_of_pair, cu_q


def _attn_ref(Q, Ks, Vs, Kc, Vc, cm, doc_of_pair, cu_q, nq, nkv, d):
    rows = Q.shape[0]
    O = np.zeros((rows, nq * d))
    L = np.zeros((rows, nq))
    Cmax = cm.shape[1]
    for p in range(len(doc_of_pair)):
        a, b = cu_q[p], cu_q[p + 1]
        dd = doc_of_pair[p]
        kc = Kc[dd * Cmax:(dd + 1) * Cmax].reshape(Cmax, nkv, d)
        vc = Vc[dd * Cmax:(dd + 1) * Cmax].reshape(Cmax, nkv, d)
        o, lse = oracle.merged_attn(Q[a:b].reshape(-1, nq, d), Ks[a:b].reshape(-1, nkv, d),
                                    Vs[a:b].reshape(-1, nkv, d), kc, vc, cm[dd])
        O[a:b] = o.reshape(b - a, nq * d)
        L[a:b] = lse
    return O, L


@pytest.mark.parametrize("name,lqs,docs_c,Cmax,nq,nkv,std,general", [
    ("g4_ragged", [1, 31, 32, 33, 100, 300], [0, 1, 31, 32, 33, 70], 70, 4, 1, 0.7, False),
    ("g4_general_mask", [45, 129, 7], [0, 0, 0], 64, 4, 1, 0.7, True),
    ("g2_gqa", [64, 65, 200, 3], [256, 100, 17, 0], 256, 8, 4, 0.7, False),
    ("g1", [130, 5, 64], [10, 129, 0], 130, 2, 2, 0.7, False),
    ("g8", [40, 97], [33, 64], 64, 8, 1, 0.7, False),
    ("g4_sharp_logits", [150, 80], [90, 40], 96, 4, 1, 3.0, False),
    ("g4_long", [512], [256], 256, 4, 1, 0.7, False),
    # the largest passage the bf16 path takes (128 key tiles: both validity words)
    ("g4_max_cmax", [40, 3], [4096, 2049], 4096, 4, 1, 0.7, False),
    ("g4_max_cmax_general_mask", [20], [0], 4096, 4, 1, 0.7, True),
])
def test_merged_attn_bf16_parity(name, lqs, docs_c, Cmax, nq, nkv, std, general):
    _announce(f"merged_attn bf16 {name}")
    d = 256
    case = _attn_case(zlib.crc32(name.encode()) % 1000 + 50, lqs, docs_c, Cmax, nq, nkv, d, True, std, general)
    Q, Ks, Vs, Kc, Vc, cm, dop, cu_q = case
    rows = Q.shape[0]
    lse = torch.empty(rows, nq, dtype=torch.float32, device="cuda")
    bf = torch.bfloat16
    O = ops.kalm_merged_attn(to_dev(Q, bf), to_dev(Ks, bf), to_dev(Vs, bf), to_dev(cu_q, torch.int32), max(lqs),
                             to_dev(Kc, bf), to_dev(Vc, bf), to_dev(cm, torch.uint8), to_dev(dop, torch.int32),
                             nq, nkv, d, lse=lse)
    torch.cuda.synchronize()
    rO, rL = _attn_ref(*case, nq, nkv, d)
    assert_close(to_np(O), rO, *BF16_TOL, f"O ({name})")
    assert_close(to_np(lse), rL, *BF16_TOL, f"lse ({name})")


@pytest.mark.parametrize("name,lqs,docs_c,Cmax,nq,nkv,d", [
    ("tiny", [16] * 8, [2, 16, 5, 9, 1, 16, 12, 7], 16, 2, 1, 32),
    ("f32_gqa_ragged", [1, 9, 40], [0, 3, 20], 20, 4, 2, 64),
])
def test_merged_attn_f32_parity(name, lqs, docs_c, Cmax, nq, nkv, d):
    _announce(f"merged_attn f32 {name}")
    case = _attn_case(7, lqs, docs_c, Cmax, nq, nkv, d, False)
    Q, Ks, Vs, Kc, Vc, cm, dop, cu_q = case
    rows = Q.shape[0]
    lse = torch.empty(rows, nq, dtype=torch.float32, device="cuda")
    f = torch.float32
    O = ops.kalm_merged_attn(to_dev(Q, f), to_dev(Ks, f), to_dev(Vs, f), to_dev(cu_q, torch.int32), max(lqs),
                             to_dev(Kc, f), to_dev(Vc, f), to_dev(cm, torch.uint8), to_dev(dop, torch.int32),
                             nq, nkv, d, lse=lse)
    torch.cuda.synchronize()
    rO, rL = _attn_ref(*case, nq, nkv, d)
    assert_close(to_np(O), rO, *F32_TOL, "O f32")
    assert_close(to_np(lse), rL, *F32_TOL, "lse f32")


@pytest.mark.parametrize("bf16", [True, False])
def test_merged_attn_final_row_mode(bf16):
    """row_mode 1: only each pair's final position, Q/O one row per pair."""
    _announce(f"merged_attn final-row mode bf16={bf16}")
    d = 256 if bf16 else 64
    lqs = [1, 33, 64, 100, 7]
    case = _attn_case(11, lqs, [0, 31, 70, 5, 64], 70, 4, 1, d, bf16)
    Q, Ks, Vs, Kc, Vc, cm, dop, cu_q = case
    P = len(lqs)
    fin = cu_q[1:] - 1
    dt = torch.bfloat16 if bf16 else torch.float32
    lse = torch.full((P, 4), -7.0, dtype=torch.float32, device="cuda")
    O = ops.kalm_merged_attn_rows(to_dev(Q[fin], dt), to_dev(Ks, dt), to_dev(Vs, dt), to_dev(cu_q, torch.int32),
                                  max(lqs), to_dev(Kc, dt), to_dev(Vc, dt), to_dev(cm, torch.uint8),
                                  to_dev(dop, torch.int32), 4, 1, d, ops.ROWS_FINAL, P, lse=lse)
    torch.cuda.synchronize()
    rO, rL = _attn_ref(*case, 4, 1, d)
    tol = BF16_TOL if bf16 else F32_TOL
    assert_close(to_np(O), rO[fin], *tol, "O final rows")
    assert_close(to_np(lse), rL[fin], *tol, "lse final rows")


@pytest.mark.parametrize("bf16", [True, False])
def test_merged_attn_shared_rows_mode(bf16):
    """row_mode 2: Q/K/V rows of each query shared by its D passages (pair
    p = query p // D, passage p % D); O in the pair layout."""
    _announce(f"merged_attn shared-rows mode bf16={bf16}")
    d = 256 if bf16 else 32
    nq, nkv, D, Cmax = 4, 1, 4, 40
    lq = np.array([5, 37, 70], np.int64)
    docs_c = [0, 3, 32, 33]
    U = int(lq.sum())
    Qu = synth.normal(21, (U, nq * d), 0.7, bf16)
    Ku = synth.normal(22, (U, nkv * d), 0.7, bf16)
    Vu = synth.normal(23, (U, nkv * d), 1.0, bf16)
    Kc = synth.normal(24, (D * Cmax, nkv * d), 0.7, bf16)
    Vc = synth.normal(25, (D * Cmax, nkv * d), 1.0, bf16)
    cm = (np.arange(Cmax)[None] < np.asarray(docs_c)[:, None]).astype(np.uint8)
    starts = np.concatenate([[0], np.cumsum(lq)])
    # pair layout: query q's D pairs back to back, each a copy of the query's rows
    idx = np.concatenate([np.arange(starts[q], starts[q + 1]) for q in range(len(lq)) for _ in range(D)])
    lens = np.repeat(lq, D)
    cu_q = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    dop = (np.arange(len(lens)) % D).astype(np.int32)
    rows = int(cu_q[-1])
    dt = torch.bfloat16 if bf16 else torch.float32
    O = ops.kalm_merged_attn_rows(to_dev(Qu, dt), to_dev(Ku, dt), to_dev(Vu, dt), to_dev(cu_q, torch.int32),
                                  int(lq.max()), to_dev(Kc, dt), to_dev(Vc, dt), to_dev(cm, torch.uint8),
                                  to_dev(dop, torch.int32), nq, nkv, d, ops.ROWS_SHARED, rows)
    torch.cuda.synchronize()
    rO, _ = _attn_ref(Qu[idx], Ku[idx], Vu[idx], Kc, Vc, cm, dop, cu_q, nq, nkv, d)
    assert_close(to_np(O), rO, *(BF16_TOL if bf16 else F32_TOL), "O shared rows")


def test_merged_attn_bad_doc_gives_nan_rows():
    _announce("merged_attn out-of-range doc")
    case = _attn_case(9, [20, 20], [5, 5], 32, 4, 1, 256, True)
    Q, Ks, Vs, Kc, Vc, cm, dop, cu_q = case
    dop = np.array([0, 7], np.int32)  # doc 7 does not exist
    bf = torch.bfloat16
    O = ops.kalm_merged_attn(to_dev(Q, bf), to_dev(Ks, bf), to_dev(Vs, bf), to_dev(cu_q, torch.int32), 20,
                             to_dev(Kc, bf), to_dev(Vc, bf), to_dev(cm, torch.uint8), to_dev(dop, torch.int32),
                             4, 1, 256)
    g = to_np(O)
    assert np.isfinite(g[:20]).all() and np.isnan(g[20:]).all()


# ------------------------------------------------------------------ a3 split at the self/cross boundary
def _self_ref(Q, Ks, Vs, cu, nq, nkv, d):
    """Oracle causal self-attention of packed sequences: the merged attention
    with no visible cross key."""
    rows = Q.shape[0]
    O = np.zeros((rows, nq * d))
    L = np.zeros((rows, nq))
    none = np.zeros((0, nkv, d))
    for i in range(len(cu) - 1):
        a, b = cu[i], cu[i + 1]
        o, lse = oracle.merged_attn(Q[a:b].reshape(-1, nq, d), Ks[a:b].reshape(-1, nkv, d),
                                    Vs[a:b].reshape(-1, nkv, d), none, none, np.zeros(0, np.uint8))
        O[a:b] = o.reshape(b - a, nq * d)
        L[a:b] = lse
    return O, L


@pytest.mark.parametrize("name,lqs,nq,nkv,bf16", [
    ("g4_ragged", [1, 31, 32, 33, 100, 300], 4, 1, True),
    ("g2_gqa", [64, 129, 5], 8, 4, True),
    ("g1_long", [512, 17], 2, 2, True),
    ("f32_gqa", [1, 9, 40, 33], 4, 2, False),
])
def test_self_attn_partial_parity(name, lqs, nq, nkv, bf16):
    _announce(f"self_attn_partial {name}")
    d = 256 if bf16 else 64
    case = _attn_case(zlib.crc32(name.encode()) % 1000 + 300, lqs, [0], 1, nq, nkv, d, bf16)
    Q, Ks, Vs, _, _, _, _, cu = case
    dt = torch.bfloat16 if bf16 else torch.float32
    O, lse = ops.kalm_self_attn_partial(to_dev(Q, dt), to_dev(Ks, dt), to_dev(Vs, dt), to_dev(cu, torch.int32),
                                        max(lqs), nq, nkv, d)
    torch.cuda.synchronize()
    assert O.dtype == torch.float32
    rO, rL = _self_ref(Q, Ks, Vs, cu, nq, nkv, d)
    tol = BF16_TOL if bf16 else F32_TOL
    assert_close(to_np(O), rO, *tol, f"O self ({name})")
    assert_close(to_np(lse), rL, *tol, f"lse self ({name})")


@pytest.mark.parametrize("name,lqs,docs_c,Cmax,nq,nkv,bf16", [
    ("g4_ragged", [1, 31, 32, 33, 100, 300], [0, 1, 31, 32, 33, 70], 70, 4, 1, True),
    ("g2_gqa_long", [64, 512, 3], [256, 100, 0], 256, 8, 4, True),
    ("f32", [1, 9, 40], [0, 3, 20], 20, 4, 2, False),
])
def test_merged_attn_resume_from_oracle_partial(name, lqs, docs_c, Cmax, nq, nkv, bf16):
    """Cross keys only, the online softmax started from the oracle's self
    partial: equals the oracle's merged attention (all rows)."""
    _announce(f"merged_attn_resume {name}")
    d = 256 if bf16 else 64
    case = _attn_case(zlib.crc32(name.encode()) % 1000 + 400, lqs, docs_c, Cmax, nq, nkv, d, bf16)
    Q, Ks, Vs, Kc, Vc, cm, dop, cu_q = case
    rows = Q.shape[0]
    sO, sL = _self_ref(Q, Ks, Vs, cu_q, nq, nkv, d)
    dt = torch.bfloat16 if bf16 else torch.float32
    f = torch.float32
    lse = torch.empty(rows, nq, dtype=f, device="cuda")
    O = ops.kalm_merged_attn_resume(to_dev(Q, dt), to_dev(sO, f), to_dev(sL, f), to_dev(cu_q, torch.int32), max(lqs),
                                    to_dev(Kc, dt), to_dev(Vc, dt), to_dev(cm, torch.uint8), to_dev(dop, torch.int32),
                                    nq, nkv, d, ops.ROWS_ALL, rows, lse=lse)
    torch.cuda.synchronize()
    rO, rL = _attn_ref(*case, nq, nkv, d)
    tol = BF16_TOL if bf16 else F32_TOL
    assert_close(to_np(O), rO, *tol, f"O resumed ({name})")
    assert_close(to_np(lse), rL, *tol, f"lse resumed ({name})")


@pytest.mark.parametrize("bf16", [True, False])
def test_merged_attn_resume_final_row_mode(bf16):
    _announce(f"merged_attn_resume final-row mode bf16={bf16}")
    d = 256 if bf16 else 64
    lqs = [1, 33, 64, 100, 7]
    case = _attn_case(12, lqs, [0, 31, 70, 5, 64], 70, 4, 1, d, bf16)
    Q, Ks, Vs, Kc, Vc, cm, dop, cu_q = case
    P = len(lqs)
    fin = cu_q[1:] - 1
    sO, sL = _self_ref(Q, Ks, Vs, cu_q, 4, 1, d)
    dt = torch.bfloat16 if bf16 else torch.float32
    f = torch.float32
    O = ops.kalm_merged_attn_resume(to_dev(Q[fin], dt), to_dev(sO[fin], f), to_dev(sL[fin], f),
                                    to_dev(cu_q, torch.int32), max(lqs), to_dev(Kc, dt), to_dev(Vc, dt),
                                    to_dev(cm, torch.uint8), to_dev(dop, torch.int32), 4, 1, d, ops.ROWS_FINAL, P)
    torch.cuda.synchronize()
    rO, _ = _attn_ref(*case, 4, 1, d)
    assert_close(to_np(O), rO[fin], *(BF16_TOL if bf16 else F32_TOL), "O resumed final rows")


@pytest.mark.parametrize("bf16", [True, False])
def test_self_partial_then_resume_shared_rows(bf16):
    """The first-layer reuse: each query's causal self-attention computed once
    (kalm_self_attn_partial over the per-query packing that kalm_pair_layout
    gives with one passage), then every pair finished from it with its
    passage's cross keys (shared rows); equals the oracle's merged attention
    of every pair."""
    _announce(f"self partial + resume shared rows bf16={bf16}")
    d = 256 if bf16 else 32
    nq, nkv, D, Cmax = 4, 1, 5, 40
    lq = np.array([5, 37, 70, 1], np.int64)
    docs_c = [0, 3, 32, 33, 40]
    U = int(lq.sum())
    Qu = synth.normal(31, (U, nq * d), 0.7, bf16)
    Ku = synth.normal(32, (U, nkv * d), 0.7, bf16)
    Vu = synth.normal(33, (U, nkv * d), 1.0, bf16)
    Kc = synth.normal(34, (D * Cmax, nkv * d), 0.7, bf16)
    Vc = synth.normal(35, (D * Cmax, nkv * d), 1.0, bf16)
    cm = (np.arange(Cmax)[None] < np.asarray(docs_c)[:, None]).astype(np.uint8)
    Kc.reshape(D, Cmax, -1)[cm == 0] = np.nan
    Vc.reshape(D, Cmax, -1)[cm == 0] = np.nan
    starts = np.concatenate([[0], np.cumsum(lq)])
    idx = np.concatenate([np.arange(starts[q], starts[q + 1]) for q in range(len(lq)) for _ in range(D)])
    lq_d = to_dev(lq.astype(np.int32), torch.int32)
    n_q = len(lq)
    P = n_q * D
    rows = int(D * U)
    cu_q = torch.empty(P + 1, dtype=torch.int32, device="cuda")
    dop = torch.empty(P, dtype=torch.int32, device="cuda")
    fin = torch.empty(P, dtype=torch.int32, device="cuda")
    lib = ops.load()
    ops._check("kalm_pair_layout", lib.kalm_pair_layout(ops._ptr(lq_d), n_q, D, ops._ptr(cu_q), ops._ptr(dop),
                                                         ops._ptr(fin), None, rows, None, None, None))
    cu_s = torch.empty(n_q + 1, dtype=torch.int32, device="cuda")
    dop1 = torch.empty(n_q, dtype=torch.int32, device="cuda")
    fin1 = torch.empty(n_q, dtype=torch.int32, device="cuda")
    ops._check("kalm_pair_layout", lib.kalm_pair_layout(ops._ptr(lq_d), n_q, 1, ops._ptr(cu_s), ops._ptr(dop1),
                                                         ops._ptr(fin1), None, U, None, None, None))
    dt = torch.bfloat16 if bf16 else torch.float32
    Qd, Kd, Vd = to_dev(Qu, dt), to_dev(Ku, dt), to_dev(Vu, dt)
    sO, sL = ops.kalm_self_attn_partial(Qd, Kd, Vd, cu_s, int(lq.max()), nq, nkv, d)
    O = ops.kalm_merged_attn_resume(Qd, sO, sL, cu_q, int(lq.max()), to_dev(Kc, dt), to_dev(Vc, dt),
                                    to_dev(cm, torch.uint8), dop, nq, nkv, d, ops.ROWS_SHARED, rows)
    torch.cuda.synchronize()
    cu_np = np.concatenate([[0], np.cumsum(np.repeat(lq, D))]).astype(np.int32)
    assert (to_np(cu_q) == cu_np).all()
    dop_np = (np.arange(P) % D).astype(np.int32)
    rO, _ = _attn_ref(Qu[idx], Ku[idx], Vu[idx], Kc, Vc, cm, dop_np, cu_np, nq, nkv, d)
    assert_close(to_np(O), rO, *(BF16_TOL if bf16 else F32_TOL), "O self partial + resume")


@pytest.mark.parametrize("bf16,reuse", [(True, True), (True, False), (False, True), (False, False)])
def test_shared_final_row_mode(bf16, reuse):
    """row_mode 3: each pair's final position only, its Q (and self partial)
    the query's last row in the per-query packing, O row p -- in one merged
    pass, or resumed from the query's self partial."""
    _announce(f"shared final-row mode bf16={bf16} reuse={reuse}")
    d = 256 if bf16 else 32
    nq, nkv, D, Cmax = 4, 1, 6, 70
    lq = np.array([5, 37, 64, 1, 100], np.int64)
    docs_c = [0, 3, 32, 33, 64, 70]
    U = int(lq.sum())
    Qu = synth.normal(41, (U, nq * d), 0.7, bf16)
    Ku = synth.normal(42, (U, nkv * d), 0.7, bf16)
    Vu = synth.normal(43, (U, nkv * d), 1.0, bf16)
    Kc = synth.normal(44, (D * Cmax, nkv * d), 0.7, bf16)
    Vc = synth.normal(45, (D * Cmax, nkv * d), 1.0, bf16)
    cm = (np.arange(Cmax)[None] < np.asarray(docs_c)[:, None]).astype(np.uint8)
    Kc.reshape(D, Cmax, -1)[cm == 0] = np.nan
    Vc.reshape(D, Cmax, -1)[cm == 0] = np.nan
    n_q = len(lq)
    P = n_q * D
    lay = ops.kalm_pair_layout(to_dev(lq.astype(np.int32), torch.int32), D, rows=int(D * U))
    lay1 = ops.kalm_pair_layout(to_dev(lq.astype(np.int32), torch.int32), 1, with_h0_row=False)
    dt = torch.bfloat16 if bf16 else torch.float32
    Qd, Kd, Vd = to_dev(Qu, dt), to_dev(Ku, dt), to_dev(Vu, dt)
    args = (to_dev(Kc, dt), to_dev(Vc, dt), to_dev(cm, torch.uint8), lay["doc_of_pair"], nq, nkv, d,
            ops.ROWS_SHARED_FINAL, P)
    lse = torch.full((P, nq), -7.0, dtype=torch.float32, device="cuda")
    if reuse:
        sO, sL = ops.kalm_self_attn_partial(Qd, Kd, Vd, lay1["cu_q"], int(lq.max()), nq, nkv, d)
        O = ops.kalm_merged_attn_resume(Qd, sO, sL, lay["cu_q"], int(lq.max()), *args, lse=lse)
    else:
        O = ops.kalm_merged_attn_rows(Qd, Kd, Vd, lay["cu_q"], int(lq.max()), *args, lse=lse)
    torch.cuda.synchronize()
    # oracle: every pair's merged attention over its expanded rows, read at its final row
    starts = np.concatenate([[0], np.cumsum(lq)])
    idx = np.concatenate([np.arange(starts[q], starts[q + 1]) for q in range(n_q) for _ in range(D)])
    cu_np = np.concatenate([[0], np.cumsum(np.repeat(lq, D))]).astype(np.int32)
    dop_np = (np.arange(P) % D).astype(np.int32)
    rO, rL = _attn_ref(Qu[idx], Ku[idx], Vu[idx], Kc, Vc, cm, dop_np, cu_np, nq, nkv, d)
    fin = cu_np[1:] - 1
    tol = BF16_TOL if bf16 else F32_TOL
    assert_close(to_np(O), rO[fin], *tol, "O shared final rows")
    assert_close(to_np(lse), rL[fin], *tol, "lse shared final rows")


@pytest.mark.parametrize("name,lqs,docs_c,Cmax,nq,nkv,n_split,general", [
    ("g4_ragged_s3", [1, 31, 32, 33, 100, 300], [0, 1, 31, 32, 33, 70], 70, 4, 1, 3, False),
    ("g4_general_s4", [45, 129, 7], [0, 0, 0], 256, 4, 1, 4, True),
    ("g2_gqa_s8", [64, 65, 3], [256, 100, 17], 256, 8, 4, 8, False),
    ("g4_s1", [40, 97], [33, 64], 64, 4, 1, 1, False),
    ("g4_more_splits_than_tiles", [20, 9], [5, 64], 64, 4, 1, 7, False),
])
def test_merged_attn_split_from_oracle_partial(name, lqs, docs_c, Cmax, nq, nkv, n_split, general):
    """Cross keys in n_split shares (split-KV) merged with the oracle's self
    partial by log-sum-exp weights: equals the oracle's merged attention."""
    _announce(f"merged_attn_split {name}")
    d = 256
    case = _attn_case(zlib.crc32(name.encode()) % 1000 + 500, lqs, docs_c, Cmax, nq, nkv, d, True, 0.7, general)
    Q, Ks, Vs, Kc, Vc, cm, dop, cu_q = case
    rows = Q.shape[0]
    sO, sL = _self_ref(Q, Ks, Vs, cu_q, nq, nkv, d)
    bf, f = torch.bfloat16, torch.float32
    lse = torch.empty(rows, nq, dtype=f, device="cuda")
    ws = torch.full((ops.split_workspace_bytes(n_split, rows, nq, d) // 4,), float("nan"), dtype=f, device="cuda")
    O = ops.kalm_merged_attn_split(to_dev(Q, bf), to_dev(sO, f), to_dev(sL, f), to_dev(cu_q, torch.int32), max(lqs),
                                   to_dev(Kc, bf), to_dev(Vc, bf), to_dev(cm, torch.uint8), to_dev(dop, torch.int32),
                                   nq, nkv, d, ops.ROWS_ALL, rows, n_split, workspace=ws, lse=lse)
    torch.cuda.synchronize()
    rO, rL = _attn_ref(*case, nq, nkv, d)
    assert_close(to_np(O), rO, *BF16_TOL, f"O split ({name})")
    assert_close(to_np(lse), rL, *BF16_TOL, f"lse split ({name})")


@pytest.mark.parametrize("n_split", [1, 2, 8])
def test_merged_attn_split_shared_final_rows(n_split):
    """The one-query, many-passage case split-KV is for: final rows of the
    shared layout, self partial from kalm_self_attn_partial."""
    _announce(f"merged_attn_split shared final rows n_split={n_split}")
    d, nq, nkv, D, Cmax = 256, 4, 1, 100, 256
    lq = np.array([64], np.int64)
    rng = np.random.default_rng(77)
    docs_c = rng.integers(8, 257, D)
    U = int(lq.sum())
    Qu = synth.normal(51, (U, nq * d), 0.7, True)
    Ku = synth.normal(52, (U, nkv * d), 0.7, True)
    Vu = synth.normal(53, (U, nkv * d), 1.0, True)
    Kc = synth.normal(54, (D * Cmax, nkv * d), 0.7, True)
    Vc = synth.normal(55, (D * Cmax, nkv * d), 1.0, True)
    cm = (np.arange(Cmax)[None] < np.asarray(docs_c)[:, None]).astype(np.uint8)
    Kc.reshape(D, Cmax, -1)[cm == 0] = np.nan
    Vc.reshape(D, Cmax, -1)[cm == 0] = np.nan
    P = D
    lay = ops.kalm_pair_layout(to_dev(lq.astype(np.int32), torch.int32), D, rows=int(D * U))
    lay1 = ops.kalm_pair_layout(to_dev(lq.astype(np.int32), torch.int32), 1, with_h0_row=False)
    bf = torch.bfloat16
    Qd, Kd, Vd = to_dev(Qu, bf), to_dev(Ku, bf), to_dev(Vu, bf)
    sO, sL = ops.kalm_self_attn_partial(Qd, Kd, Vd, lay1["cu_q"], int(lq.max()), nq, nkv, d)
    O = ops.kalm_merged_attn_split(Qd, sO, sL, lay["cu_q"], int(lq.max()), to_dev(Kc, bf), to_dev(Vc, bf),
                                   to_dev(cm, torch.uint8), lay["doc_of_pair"], nq, nkv, d, ops.ROWS_SHARED_FINAL, P,
                                   n_split)
    torch.cuda.synchronize()
    idx = np.tile(np.arange(U), D)
    cu_np = np.concatenate([[0], np.cumsum(np.repeat(lq, D))]).astype(np.int32)
    dop_np = (np.arange(P) % D).astype(np.int32)
    rO, _ = _attn_ref(Qu[idx], Ku[idx], Vu[idx], Kc, Vc, cm, dop_np, cu_np, nq, nkv, d)
    assert_close(to_np(O), rO[cu_np[1:] - 1], *BF16_TOL, "O split shared final rows")


def test_merged_attn_split_bad_doc_gives_nan_rows():
    _announce("merged_attn_split out-of-range doc")
    case = _attn_case(14, [20, 20], [5, 64], 64, 4, 1, 256, True)
    Q, Ks, Vs, Kc, Vc, cm, dop, cu_q = case
    sO, sL = _self_ref(Q, Ks, Vs, cu_q, 4, 1, 256)
    dop = np.array([0, 7], np.int32)
    bf, f = torch.bfloat16, torch.float32
    O = ops.kalm_merged_attn_split(to_dev(Q, bf), to_dev(sO, f), to_dev(sL, f), to_dev(cu_q, torch.int32), 20,
                                   to_dev(Kc, bf), to_dev(Vc, bf), to_dev(cm, torch.uint8), to_dev(dop, torch.int32),
                                   4, 1, 256, ops.ROWS_ALL, 40, 2)
    g = to_np(O)
    assert np.isfinite(g[:20]).all() and np.isnan(g[20:]).all()


def test_merged_attn_resume_bad_doc_gives_nan_rows():
    _announce("merged_attn_resume out-of-range doc")
    case = _attn_case(13, [20, 20], [5, 5], 32, 4, 1, 256, True)
    Q, Ks, Vs, Kc, Vc, cm, dop, cu_q = case
    sO, sL = _self_ref(Q, Ks, Vs, cu_q, 4, 1, 256)
    dop = np.array([0, 7], np.int32)
    bf, f = torch.bfloat16, torch.float32
    O = ops.kalm_merged_attn_resume(to_dev(Q, bf), to_dev(sO, f), to_dev(sL, f), to_dev(cu_q, torch.int32), 20,
                                    to_dev(Kc, bf), to_dev(Vc, bf), to_dev(cm, torch.uint8), to_dev(dop, torch.int32),
                                    4, 1, 256, ops.ROWS_ALL, 40)
    g = to_np(O)
    assert np.isfinite(g[:20]).all() and np.isnan(g[20:]).all()


# ------------------------------------------------------------------ model-shaped layer parts
@pytest.mark.parametrize("M,H,xdt,ydt", [(1000, 1152, "f32", "bf16"), (37, 640, "f32", "f32"), (5, 64, "bf16", "bf16"),
                                         (300, 2560, "bf16", "f32")])
def test_rms_norm_parity(M, H, xdt, ydt):
    _announce(f"rms_norm M={M} H={H} {xdt}->{ydt}")
    t = {"f32": torch.float32, "bf16": torch.bfloat16}
    x = synth.normal(61, (M, H), 1.5, xdt == "bf16")
    x[3 % M] *= 40.0  # one large row
    if xdt == "bf16":
        x = synth.round_to_bf16(x)  # the device input is exactly what the oracle sees
    w = 1.0 + synth.normal(62, (H,), 0.1, ydt == "bf16")
    w = synth.round_to_bf16(w) if ydt == "bf16" else w
    y = ops.kalm_rms_norm(to_dev(x, t[xdt]), to_dev(w, t[ydt]), 1e-6, y_dtype=t[ydt])
    torch.cuda.synchronize()
    ref = oracle.rms_norm(x, w, 1e-6)
    assert_close(to_np(y), ref, *(BF16_TOL if ydt == "bf16" else F32_TOL), "rms_norm")


@pytest.mark.parametrize("bf16,mode", [(True, 0), (False, 0), (True, 1), (False, 1)])
def test_rope_parity(bf16, mode):
    _announce(f"rope bf16={bf16} mode={mode}")
    nq, nkv, d = 4, 2, 256 if bf16 else 64
    lens = np.array([1, 31, 130, 512, 7], np.int64)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    rows = int(lens.sum()) if mode == 0 else len(lens)
    ld = (nq + 2 * nkv) * d
    X = synth.normal(63, (rows, ld), 1.0, bf16)
    dt = torch.bfloat16 if bf16 else torch.float32
    Xd = to_dev(X, dt)
    ops.kalm_rope(Xd, 0, nq, d, to_dev(cu, torch.int32), int(lens.max()), mode, 10000.0)
    ops.kalm_rope(Xd, nq * d, nkv, d, to_dev(cu, torch.int32), int(lens.max()), mode, 10000.0)
    torch.cuda.synchronize()
    pos = np.concatenate([np.arange(n) for n in lens]) if mode == 0 else lens - 1
    ref = X.astype(np.float64).copy()
    ref[:, :nq * d] = oracle.rope(X[:, :nq * d].reshape(rows, nq, d), pos, 10000.0).reshape(rows, -1)
    ref[:, nq * d:(nq + nkv) * d] = oracle.rope(X[:, nq * d:(nq + nkv) * d].reshape(rows, nkv, d), pos,
                                                10000.0).reshape(rows, -1)
    got = to_np(Xd)
    assert_close(got, ref, *(BF16_TOL if bf16 else F32_TOL), "rope")
    # the V columns are not touched
    assert np.array_equal(got[:, (nq + nkv) * d:], X[:, (nq + nkv) * d:].astype(np.float64))


@pytest.mark.parametrize("M,I,bf16", [(1000, 1536, True), (33, 64, False), (7, 4, True)])
def test_gated_gelu_parity(M, I, bf16):
    _announce(f"gated_gelu M={M} I={I} bf16={bf16}")
    Y = synth.normal(64, (M, 2 * I), 2.0, bf16)
    dt = torch.bfloat16 if bf16 else torch.float32
    A = ops.kalm_gated_gelu(to_dev(Y, dt))
    torch.cuda.synchronize()
    ref = oracle.gated_gelu(Y[:, :I], Y[:, I:])
    assert_close(to_np(A), ref, *(BF16_TOL if bf16 else F32_TOL), "gated_gelu")


@pytest.mark.parametrize("M,K,I", [(300, 200, 128), (513, 640, 384), (1, 64, 256), (1100, 1152, 768),
                                   # more tiles than workgroups: the persistent loop carries its copy
                                   # ring across tiles (with a K tail)
                                   (20000, 1000, 1536)])
def test_linear_gated_gelu_parity(M, K, I):
    # the fused gate/up projection + activation against fp64 products of the
    # same bf16 operands: ragged M, a K tail (K % 64 != 0), several 128-unit blocks
    _announce(f"linear_gated_gelu M={M} K={K} I={I}")
    X = synth.normal(70, (M, K), 1.0, True)
    Wg = synth.normal(71, (I, K), 1.0 / np.sqrt(K), True)
    Wu = synth.normal(72, (I, K), 1.0 / np.sqrt(K), True)
    bf = torch.bfloat16
    A = ops.kalm_linear_gated_gelu(to_dev(X, bf), to_dev(Wg, bf), to_dev(Wu, bf))
    torch.cuda.synchronize()
    Xd = X.astype(np.float64)
    ref = oracle.gated_gelu(Xd @ Wg.astype(np.float64).T, Xd @ Wu.astype(np.float64).T)
    assert_close(to_np(A), ref, *BF16_TOL, "linear_gated_gelu")


# ------------------------------------------------------------------ empty inputs
def test_zero_sized_calls_are_valid_noops():
    """Every entry point accepts an empty batch (no pairs, rows, passages or
    sequences) and returns OK without touching its outputs."""
    _announce("zero-sized calls")
    dev = "cuda"
    bf, f, i32, u8 = torch.bfloat16, torch.float32, torch.int32, torch.uint8
    lay = ops.kalm_pair_layout(torch.zeros(0, dtype=i32, device=dev), 5, rows=0)
    torch.cuda.synchronize()
    assert lay["cu_q"].cpu().tolist() == [0] and lay["cu_u"].cpu().tolist() == [0]
    pooled, cm, nc = ops.kalm_chunk_pool(torch.zeros(0, 8, 64, dtype=bf, device=dev),
                                         torch.zeros(0, 8, dtype=u8, device=dev))
    assert pooled.shape[0] == 0
    W = torch.zeros(512, 64, dtype=bf, device=dev)
    assert ops.kalm_cross_kv(pooled, cm, W).shape[0] == 0
    X = torch.zeros(0, 64, dtype=bf, device=dev)
    assert ops.kalm_linear(X, W).shape[0] == 0
    Yf = torch.full((4, 512), 7.0, dtype=f, device=dev)
    ops.kalm_linear_residual(X, W, Yf, None, Y=Yf[:0])
    Q = torch.zeros(0, 1024, dtype=bf, device=dev)
    KV = torch.zeros(0, 256, dtype=bf, device=dev)
    Kc = torch.zeros(4 * 16, 256, dtype=bf, device=dev)
    cm4 = torch.ones(4, 16, dtype=u8, device=dev)
    cu0 = torch.zeros(1, dtype=i32, device=dev)
    dop0 = torch.zeros(0, dtype=i32, device=dev)
    assert ops.kalm_merged_attn(Q, KV, KV, cu0, 0, Kc, Kc, cm4, dop0, 4, 1, 256).shape[0] == 0
    o_s, l_s = ops.kalm_self_attn_partial(Q, KV, KV, cu0, 0, 4, 1, 256)
    assert o_s.shape[0] == 0
    assert ops.kalm_merged_attn_resume(Q, o_s, l_s, cu0, 0, Kc, Kc, cm4, dop0, 4, 1, 256, ops.ROWS_ALL,
                                       0).shape[0] == 0
    assert ops.kalm_merged_attn_split(Q, o_s, l_s, cu0, 0, Kc, Kc, cm4, dop0, 4, 1, 256, ops.ROWS_ALL, 0,
                                      4).shape[0] == 0
    outs = ops.kalm_yesno_score(torch.zeros(3, 64, dtype=f, device=dev), dop0, torch.zeros(2, 64, dtype=f, device=dev))
    assert all(o.numel() == 0 for o in outs)
    idx, sc = ops.kalm_rank_topn(torch.zeros(0, 10, dtype=f, device=dev), 3)
    assert idx.shape == (0, 3)
    assert ops.kalm_gather_rows(torch.zeros(3, 64, dtype=f, device=dev), dop0).shape[0] == 0
    assert ops.kalm_rms_norm(torch.zeros(0, 64, dtype=f, device=dev), torch.ones(64, dtype=f, device=dev)).shape[0] == 0
    Xr = torch.full((2, 64), 3.0, dtype=f, device=dev)
    ops.kalm_rope(Xr, 0, 2, 32, cu0, 0)
    assert ops.kalm_gated_gelu(torch.zeros(0, 64, dtype=bf, device=dev)).shape[0] == 0
    wgu = torch.zeros(128, 64, dtype=bf, device=dev)
    assert ops.kalm_linear_gated_gelu(torch.zeros(0, 64, dtype=bf, device=dev), wgu, wgu).shape == (0, 128)
    torch.cuda.synchronize()
    assert (Yf == 7.0).all() and (Xr == 3.0).all()


# ------------------------------------------------------------------ a4 score
@pytest.mark.parametrize("H,hb,wb", [(640, False, True), (1152, True, True), (64, False, False)])
def test_yesno_score_parity(H, hb, wb):
    _announce(f"yesno H={H}")
    rows, P = 300, 57
    h = synth.normal(40 + H, (rows, H), 1.0, hb)
    h[:3] *= 32.0  # large margins (a power of two keeps bf16 values exact)
    w = synth.normal(41 + H, (2, H), 0.02 if H > 64 else 1.0, wb)
    fr = synth.integers(42, 0, rows - 1, P)
    fr[:3] = [0, 1, 2]
    y, n, m, s = ops.kalm_yesno_score(to_dev(h, torch.bfloat16 if hb else torch.float32), to_dev(fr, torch.int32),
                                      to_dev(w, torch.bfloat16 if wb else torch.float32))
    torch.cuda.synchronize()
    ref = oracle.yesno_score(h[fr], w)
    for got, k in ((y, "yes"), (n, "no"), (m, "margin")):
        assert_close(to_np(got), ref[k], 1e-4, 1e-4, k)
    assert_close(to_np(s), ref["score"], 1e-5, 1e-4, "score")


# ------------------------------------------------------------------ a5 gather
def test_gather_rows_exact():
    _announce("gather_rows")
    src = synth.normal(50, (37, 1152), 1.0, False)
    idx = synth.integers(51, 0, 36, 500)
    idx[7] = 37  # out of range -> NaN row
    dst_b = torch.empty(500, 1152, dtype=torch.bfloat16, device="cuda")
    dst = ops.kalm_gather_rows(to_dev(src, torch.float32), to_dev(idx, torch.int32), dst_bf16=dst_b)
    torch.cuda.synchronize()
    g = dst.cpu().numpy()
    ok = np.arange(500) != 7
    assert np.array_equal(g[ok], src[idx[ok]])
    assert np.isnan(g[7]).all()
    assert torch.equal(dst_b.cpu()[torch.from_numpy(ok)], torch.from_numpy(src[idx[ok]]).to(torch.bfloat16))


# ------------------------------------------------------------------ ranking above the score
@pytest.mark.parametrize("Qn,D,top_n", [(5, 100, 10), (3, 100, 100), (2, 4096, 64), (1, 1, 1)])
def test_rank_topn_exact(Qn, D, top_n):
    _announce(f"rank_topn Q={Qn} D={D} top_n={top_n}")
    rng = np.random.default_rng(D + top_n)
    sc = (np.round(rng.random((Qn, D)) * 16) / 16).astype(np.float32)   # many equal scores
    if D > 3:
        sc[0, [1, D // 2, D - 1]] = np.nan
    idx, val = ops.kalm_rank_topn(to_dev(sc, torch.float32), top_n)
    r_idx, r_val = oracle.rank_topn(sc.astype(np.float64), top_n)
    assert np.array_equal(to_np(idx), r_idx)
    assert np.array_equal(to_np(val), r_val, equal_nan=True)


def test_rerank_records_follow_the_ranking():
    _announce("rerank records")
    from encoder_decoder_document_amd import rerank
    sc = np.array([0.2, 0.9, 0.2, 0.7, 0.5, 0.5], np.float32)       # 2 queries x 3 passages
    out = rerank.rerank(to_dev(sc, torch.float32), 3, 2)
    assert out == [[{"index": 1, "relevance_score": float(np.float32(0.9))},
                    {"index": 0, "relevance_score": float(np.float32(0.2))}],
                   [{"index": 0, "relevance_score": float(np.float32(0.7))},
                    {"index": 1, "relevance_score": float(np.float32(0.5))}]]

