"""Pins of the CPU oracle against things other than itself.

Each test ties an oracle function to a hand-worked example (tests/golden), a
closed form, an invariant, a library routine (torch fp64 SDPA, scipy, numpy)
or brute-force loops on tiny inputs, chosen so that a plausible mistake (a
dropped term, a wrong index or sign, a transposed operand, a wrong divisor)
fails at least one of them.  CPU only.
"""
import dataclasses
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from encoder_decoder_document_amd import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ------------------------------------------------------------------ pooling
def test_pool_worked_example():
    g = _gold("pool_worked_example.json")
    x = np.asarray(g["x"], dtype=np.float64)[:, :, None]
    pooled, cm, nc = oracle.chunk_pool(x, np.asarray(g["token_mask"], np.uint8), g["chunk"])
    np.testing.assert_array_equal(pooled[:, :, 0], np.asarray(g["pooled"]))
    np.testing.assert_array_equal(cm, np.asarray(g["chunk_mask"]))
    np.testing.assert_array_equal(nc, np.asarray(g["n_chunks"]))


@pytest.mark.parametrize("T", [1, 5, 63, 64, 1024])
def test_pool_counts_closed_form(T):
    rng = np.random.default_rng(T)
    D = 40
    lens = rng.integers(0, T + 1, size=D)
    mask = (np.arange(T)[None] < lens[:, None]).astype(np.uint8)
    x = rng.standard_normal((D, T, 2))
    _, cm, nc = oracle.chunk_pool(x, mask, 4)
    np.testing.assert_array_equal(nc, -(-lens // 4))
    np.testing.assert_array_equal(cm, (np.arange(cm.shape[1])[None] < nc[:, None]).astype(np.uint8))
    assert cm.shape[1] == -(-T // 4)


def test_pool_constant_chunks_exact():
    rng = np.random.default_rng(1)
    D, T, H = 6, 37, 16
    lens = rng.integers(1, T + 1, size=D)
    mask = (np.arange(T)[None] < lens[:, None]).astype(np.uint8)
    const = rng.standard_normal((D, -(-T // 4), H)).astype(np.float32).astype(np.float64)
    x = np.repeat(const, 4, axis=1)[:, :T]
    pooled, cm, _ = oracle.chunk_pool(x, mask, 4)
    assert np.array_equal(pooled[cm == 1], const[cm == 1])


def test_pool_partial_chunk_single_token_and_divisor():
    # len = 4k+1: the last chunk holds one valid token and must equal it (a /4
    # divisor would give a quarter of it); len = 4k+3: mean of three.
    rng = np.random.default_rng(2)
    H = 8
    x = rng.standard_normal((2, 12, H))
    mask = np.zeros((2, 12), np.uint8)
    mask[0, :9] = 1
    mask[1, :11] = 1
    pooled, _, nc = oracle.chunk_pool(x, mask, 4)
    assert np.array_equal(pooled[0, 2], x[0, 8])
    np.testing.assert_allclose(pooled[1, 2], (x[1, 8] + x[1, 9] + x[1, 10]) / 3, rtol=0, atol=1e-15)
    assert list(nc) == [3, 3]


def test_pool_chunk1_identity_and_chunk_ge_T_is_mean():
    rng = np.random.default_rng(3)
    D, T, H = 5, 23, 7
    lens = rng.integers(1, T + 1, size=D)
    mask = (np.arange(T)[None] < lens[:, None]).astype(np.uint8)
    x = rng.standard_normal((D, T, H))
    p1, cm1, _ = oracle.chunk_pool(x, mask, 1)
    assert np.array_equal(p1[cm1 == 1], x[mask == 1])
    pT, cmT, ncT = oracle.chunk_pool(x, mask, 64)
    assert pT.shape[1] == 1 and list(ncT) == [1] * D
    for d in range(D):
        np.testing.assert_allclose(pT[d, 0], np.mean(x[d, :lens[d]], axis=0), rtol=1e-14, atol=1e-15)


def test_pool_nan_padding_never_leaks_and_general_masks():
    rng = np.random.default_rng(4)
    D, T, H = 7, 30, 5
    mask = (rng.random((D, T)) < 0.5).astype(np.uint8)
    x = rng.standard_normal((D, T, H))
    x[mask == 0] = np.nan
    pooled, cm, nc = oracle.chunk_pool(x, mask, 4)
    assert np.isfinite(pooled).all()
    # brute force, pure Python loops
    for d in range(D):
        n = 0
        for c in range(pooled.shape[1]):
            vals = [x[d, t] for t in range(4 * c, min(T, 4 * c + 4)) if mask[d, t]]
            if vals:
                n += 1
                ref = [sum(v[h] for v in vals) / len(vals) for h in range(H)]
                assert cm[d, c] == 1
                np.testing.assert_allclose(pooled[d, c], ref, rtol=1e-14, atol=1e-15)
            else:
                assert cm[d, c] == 0 and not pooled[d, c].any()
        assert nc[d] == n


# ------------------------------------------------------------------ cross K/V
def test_cross_kv_bruteforce_orientation():
    rng = np.random.default_rng(5)
    C, H, N = 3, 4, 6
    p = rng.standard_normal((C, H))
    Wk = rng.standard_normal((N, H))
    Wv = rng.standard_normal((N, H))
    K, V = oracle.cross_kv(p, Wk, Wv)
    for c in range(C):
        for n in range(N):
            assert math.isclose(K[c, n], sum(p[c, k] * Wk[n, k] for k in range(H)), rel_tol=1e-13, abs_tol=1e-13)
            assert math.isclose(V[c, n], sum(p[c, k] * Wv[n, k] for k in range(H)), rel_tol=1e-13, abs_tol=1e-13)


def test_cross_kv_linearity_ties_pool_and_projection():
    # W mean(x) = mean(W x): pooling then projecting equals projecting tokens then pooling.
    rng = np.random.default_rng(6)
    D, T, H, N = 4, 19, 8, 12
    lens = rng.integers(0, T + 1, size=D)
    mask = (np.arange(T)[None] < lens[:, None]).astype(np.uint8)
    x = rng.standard_normal((D, T, H))
    Wk = rng.standard_normal((N, H))
    Wv = rng.standard_normal((N, H))
    pooled, cm, _ = oracle.chunk_pool(x, mask, 4)
    K, V = oracle.cross_kv(pooled, Wk, Wv)
    xk = np.einsum("dth,nh->dtn", x, Wk)
    pk, _, _ = oracle.chunk_pool(xk, mask, 4)
    np.testing.assert_allclose(K, pk, rtol=1e-12, atol=1e-12)
    assert not K[cm == 0].any() and not V[cm == 0].any()


# ------------------------------------------------------------------ merged attention
def _torch_sdpa_merged(Q, Ks, Vs, Kc, Vc, cmask, scale):
    """Independent formulation: torch's fp64 SDPA with an explicit boolean mask
    over the concatenated KV and GQA by repeating KV heads."""
    Q = torch.as_tensor(Q, dtype=torch.float64)
    Lq, nq, d = Q.shape
    nkv = Ks.shape[1]
    K = torch.cat([torch.as_tensor(Ks, dtype=torch.float64), torch.as_tensor(Kc, dtype=torch.float64)], 0)
    V = torch.cat([torch.as_tensor(Vs, dtype=torch.float64), torch.as_tensor(Vc, dtype=torch.float64)], 0)
    K = K.repeat_interleave(nq // nkv, dim=1).permute(1, 0, 2)
    V = V.repeat_interleave(nq // nkv, dim=1).permute(1, 0, 2)
    C = Kc.shape[0]
    allow = torch.cat([torch.ones(Lq, Lq, dtype=torch.bool).tril(),
                       torch.as_tensor(np.asarray(cmask) != 0)[None, :].expand(Lq, C)], 1)
    o = torch.nn.functional.scaled_dot_product_attention(Q.permute(1, 0, 2), K, V, attn_mask=allow, scale=scale)
    return o.permute(1, 0, 2).numpy()


def test_attn_worked_example():
    g = _gold("attn_worked_example.json")
    O, lse = oracle.merged_attn(np.asarray(g["Q"]), np.asarray(g["Ks"]), np.asarray(g["Vs"]),
                                np.asarray(g["Kc"]), np.asarray(g["Vc"]), np.asarray(g["chunk_mask"]),
                                scale=g["scale"])
    np.testing.assert_allclose(O, np.asarray(g["O"]), rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(lse, np.asarray(g["lse"]), rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("Lq,C,nq,nkv,d", [(1, 5, 1, 1, 8), (7, 9, 4, 1, 16), (13, 4, 8, 4, 8), (5, 0, 2, 2, 4)])
def test_attn_matches_torch_sdpa_fp64(Lq, C, nq, nkv, d):
    rng = np.random.default_rng(Lq * 100 + C)
    Q = rng.standard_normal((Lq, nq, d))
    Ks, Vs = rng.standard_normal((2, Lq, nkv, d))
    Kc, Vc = rng.standard_normal((2, C, nkv, d))
    cmask = (rng.random(C) < 0.6).astype(np.uint8)
    if C:
        cmask[0] = 1
    O, _ = oracle.merged_attn(Q, Ks, Vs, Kc, Vc, cmask)
    ref = _torch_sdpa_merged(Q, Ks, Vs, Kc, Vc, cmask, 1.0 / math.sqrt(d))
    np.testing.assert_allclose(O, ref, rtol=1e-12, atol=1e-12)


def test_attn_two_pass_equals_lse_merge_of_self_and_cross_partials():
    # Brute-force softmax over the concatenation == log-sum-exp merge of a
    # causal self-only partial and a cross-only partial, both from torch.
    rng = np.random.default_rng(7)
    Lq, C, d = 11, 6, 16
    Q = rng.standard_normal((Lq, 1, d))
    Ks, Vs = rng.standard_normal((2, Lq, 1, d))
    Kc, Vc = rng.standard_normal((2, C, 1, d))
    cmask = np.array([1, 0, 1, 1, 0, 1], np.uint8)
    scale = 1.0 / math.sqrt(d)
    O, lse = oracle.merged_attn(Q, Ks, Vs, Kc, Vc, cmask)
    q = torch.as_tensor(Q[:, 0])
    s_self = (q @ torch.as_tensor(Ks[:, 0]).T) * scale
    s_self = s_self.masked_fill(~torch.ones(Lq, Lq, dtype=torch.bool).tril(), -math.inf)
    lse_s = torch.logsumexp(s_self, 1)
    o_s = torch.nn.functional.scaled_dot_product_attention(
        q[None], torch.as_tensor(Ks[:, 0])[None], torch.as_tensor(Vs[:, 0])[None], is_causal=True, scale=scale)[0]
    kc = torch.as_tensor(Kc[cmask == 1, 0])
    vc = torch.as_tensor(Vc[cmask == 1, 0])
    lse_c = torch.logsumexp((q @ kc.T) * scale, 1)
    o_c = torch.nn.functional.scaled_dot_product_attention(q[None], kc[None], vc[None], scale=scale)[0]
    L = torch.logaddexp(lse_s, lse_c)
    merged = torch.exp(lse_s - L)[:, None] * o_s + torch.exp(lse_c - L)[:, None] * o_c
    np.testing.assert_allclose(O[:, 0], merged.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse[:, 0], L.numpy(), rtol=1e-12, atol=1e-12)
    # the helper used to state the split agrees with the same partials
    o_s2, lse_s2 = oracle.merged_attn_partial(Q[:, 0], Ks[:, 0], Vs[:, 0], np.tril(np.ones((Lq, Lq), bool)), scale)
    np.testing.assert_allclose(o_s2, o_s.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse_s2, lse_s.numpy(), rtol=1e-12, atol=1e-12)


def test_attn_fully_masked_cross_is_causal_self_attention():
    rng = np.random.default_rng(8)
    Lq, C, nq, d = 9, 5, 4, 8
    Q = rng.standard_normal((Lq, nq, d))
    Ks, Vs = rng.standard_normal((2, Lq, 1, d))
    Kc, Vc = rng.standard_normal((2, C, 1, d)) * 50
    O, _ = oracle.merged_attn(Q, Ks, Vs, Kc, Vc, np.zeros(C, np.uint8))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.as_tensor(Q).permute(1, 0, 2), torch.as_tensor(Ks).permute(1, 0, 2).expand(nq, Lq, d),
        torch.as_tensor(Vs).permute(1, 0, 2).expand(nq, Lq, d), is_causal=True)
    np.testing.assert_allclose(O, ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)
    # row 0 sees exactly one key: its own value comes back exactly
    assert np.array_equal(O[0], np.repeat(Vs[0], nq, axis=0))


def test_attn_cross_permutation_and_gqa_replication_invariance():
    rng = np.random.default_rng(9)
    Lq, C, nq, nkv, d = 6, 8, 4, 2, 8
    Q = rng.standard_normal((Lq, nq, d))
    Ks, Vs = rng.standard_normal((2, Lq, nkv, d))
    Kc, Vc = rng.standard_normal((2, C, nkv, d))
    cmask = np.array([1, 1, 0, 1, 0, 1, 1, 1], np.uint8)
    O, lse = oracle.merged_attn(Q, Ks, Vs, Kc, Vc, cmask)
    perm = rng.permutation(C)
    O2, lse2 = oracle.merged_attn(Q, Ks, Vs, Kc[perm], Vc[perm], cmask[perm])
    np.testing.assert_allclose(O2, O, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(lse2, lse, rtol=1e-13, atol=1e-13)
    rep = lambda a: np.repeat(a, nq // nkv, axis=1)
    O3, _ = oracle.merged_attn(Q, rep(Ks), rep(Vs), rep(Kc), rep(Vc), cmask)
    np.testing.assert_allclose(O3, O, rtol=1e-13, atol=1e-13)
    # a wrong GQA mapping (h % nkv) would differ here
    assert not np.allclose(O[:, 1], oracle.merged_attn(Q[:, [1]], Ks[:, [1]], Vs[:, [1]], Kc[:, [1]], Vc[:, [1]], cmask)[0][:, 0])


# ------------------------------------------------------------------ score
def test_score_worked_example():
    g = _gold("score_worked_example.json")
    out = oracle.yesno_score(np.asarray(g["h_final"], float), np.asarray(g["w_yesno"]))
    for k in ("yes", "no", "margin", "score"):
        np.testing.assert_allclose(out[k], np.asarray(g[k]), rtol=1e-15, atol=1e-15)


def test_score_softmax_sigmoid_identity_and_library():
    margins = np.concatenate([np.linspace(-100, 100, 2001), [0.0, 745.0, -745.0]])
    rng = np.random.default_rng(10)
    y = rng.standard_normal(margins.size) * 3
    n = y - margins
    H = 2
    h = np.stack([y, n], 1)
    out = oracle.yesno_score(h, np.eye(H))
    np.testing.assert_allclose(out["score"], scipy.special.expit(margins), rtol=1e-13, atol=1e-300)
    np.testing.assert_allclose(out["softmax2"], scipy.special.softmax(np.stack([y, n], 1), axis=1)[:, 0],
                               rtol=1e-12, atol=1e-300)
    np.testing.assert_allclose(out["score"], out["softmax2"], rtol=1e-12, atol=1e-300)
    assert out["score"][np.argmin(np.abs(margins))] == 0.5
    assert np.isfinite(out["score"]).all()
    np.testing.assert_allclose(out["score"] + oracle.yesno_score(np.stack([n, y], 1), np.eye(2))["score"], 1.0,
                               rtol=0, atol=1e-15)


# ------------------------------------------------------------------ layout
def test_pair_layout_closed_form():
    lq = [3, 1, 4]
    D = 2
    lay = oracle.pair_layout(lq, D)
    assert list(lay["cu_q"]) == [0, 3, 6, 7, 8, 12, 16]
    assert list(lay["doc_of_pair"]) == [0, 1, 0, 1, 0, 1]
    assert list(lay["query_of_pair"]) == [0, 0, 1, 1, 2, 2]
    assert list(lay["final_row"]) == [2, 5, 6, 7, 11, 15]
    assert list(lay["h0_row"]) == [0, 1, 2, 0, 1, 2, 3, 3, 4, 5, 6, 7, 4, 5, 6, 7]
    assert list(lay["h0_final"]) == [2, 2, 3, 3, 7, 7]
    assert list(lay["cu_u"]) == [0, 3, 4, 8]
    # the final position's query row is the query row of the pair's final row
    assert list(lay["h0_final"]) == [int(lay["h0_row"][f]) for f in lay["final_row"]]


# ------------------------------------------------------------------ rounding helpers
def test_round_bf16_against_bit_truncation_definition():
    rng = np.random.default_rng(11)
    a = np.concatenate([rng.standard_normal(20000) * 10 ** rng.uniform(-6, 6, 20000),
                        [0.0, -0.0, 1.0, 1.00390625, 1.005859375, 1.0078125 * 3]])
    r = oracle.round_bf16(a)
    # bf16 values have at most 8 significant bits
    m, _ = np.frexp(r)
    assert np.array_equal(m * 256, np.rint(m * 256))
    # nearest: no other 8-bit value is closer; ties (1 + 2^-8) go to even (1.0)
    ulp = np.ldexp(1.0, np.frexp(np.abs(a))[1] - 8)
    assert (np.abs(r - a) <= ulp / 2 + 1e-300).all()
    assert oracle.round_bf16(1.00390625) == 1.0
    assert oracle.round_bf16(1.005859375) == 1.0078125  # 3/4 of an ulp above 1: rounds up
    # agrees with torch's bf16 conversion on float32-representable input
    a32 = a.astype(np.float32)
    np.testing.assert_array_equal(oracle.round_bf16(a32.astype(np.float64)),
                                  torch.as_tensor(a32).to(torch.bfloat16).to(torch.float64).numpy())


# Every finite non-negative bf16 value, in increasing order: the upper 16
# bits of a float32 (0x0000 .. 0x7F7F), each pattern read as a number.
_BF16_BITS = np.arange(0, 0x7F80, dtype=np.uint32)
_BF16_VALS = (_BF16_BITS << 16).view(np.float32).astype(np.float64)


def _bf16_nearest_by_table(a):
    """Nearest bf16 value by search over the table of all bf16 values: the
    closer neighbour, the one with an even bit pattern on a tie, +-inf past
    the midpoint between the largest finite value and 2^128."""
    a = np.asarray(a, dtype=np.float64)
    x = np.abs(a)
    j = np.clip(np.searchsorted(_BF16_VALS, x), 1, len(_BF16_VALS) - 1)
    lo, hi = _BF16_VALS[j - 1], _BF16_VALS[j]
    dlo, dhi = x - lo, hi - x
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (_BF16_BITS[j] % 2 == 0))
    r = np.where(pick_hi, hi, lo)
    r = np.where(x == 0, 0.0, r)
    top = _BF16_VALS[-1]
    mid_inf = top + (top - _BF16_VALS[-2]) / 2          # halfway to 2^128; ties go to 2^128 (even) = inf
    r = np.where(x >= mid_inf, np.inf, np.where(x > top, top, r))
    return np.where(np.isnan(a), np.nan, np.copysign(r, a))


def test_round_bf16_full_range_against_the_table_of_all_values():
    # normal, subnormal (below 2^-126: multiples of 2^-133) and overflowing
    # inputs, and exact midpoints between neighbouring bf16 values
    rng = np.random.default_rng(12)
    a = rng.standard_normal(40000) * 10.0 ** rng.uniform(-45, 38.6, 40000)
    k = rng.integers(0, len(_BF16_VALS) - 1, 4000)
    mids = (_BF16_VALS[k] + _BF16_VALS[k + 1]) / 2
    sub = rng.integers(0, 1 << 8, 2000) * 2.0 ** -134          # subnormal grid and its midpoints
    top = _BF16_VALS[-1]
    special = np.array([0.0, -0.0, top, -top, top + (top - _BF16_VALS[-2]) / 2, 2.0 ** 128, 1e39, -1e39,
                        2.0 ** -133, 2.0 ** -134, 3 * 2.0 ** -134, 2.0 ** -126, 2.0 ** -126 - 2.0 ** -134,
                        np.inf, -np.inf])
    a = np.concatenate([a, mids, -mids, sub, -sub, special])
    got = oracle.round_bf16(a)
    ref = _bf16_nearest_by_table(a)
    np.testing.assert_array_equal(got, ref)
    assert np.array_equal(np.signbit(got), np.signbit(ref))
    assert np.isnan(oracle.round_bf16(np.nan))


# ------------------------------------------------------------------ stack: mirror-mode storage points
# One pair, one layer, one head (nq = nkv = 1, d = H), weights chosen so the
# attention reduces to a closed form: one visible key (its value), uniform
# weights (Wq = 0: the mean of the visible values) or two keys (a logistic
# weight).  Storage rounding is applied with the table search above, fp32
# storage with a float32 cast; the oracle's mirror mode must match exactly.
def _bf(a):
    return _bf16_nearest_by_table(a)


def _f32(a):
    return np.asarray(a, dtype=np.float64).astype(np.float32).astype(np.float64)


def _one_pair(h0, x_doc, mask_doc, W):
    Lq, H = h0.shape
    T = x_doc.shape[0]
    sh = synth.Shape("closed_form", 1, 1, T, H, 1, 1, H, 1, "bf16", ("list", [int(mask_doc.sum())], 0),
                     ("list", [Lq], 0))
    inp = dict(shape=sh, x=x_doc[None].astype(np.float32), token_mask=mask_doc[None].astype(np.uint8),
               lq=np.array([Lq], np.int32), h0=h0.astype(np.float32), layers=[W],
               w_yesno=np.ones((2, H), np.float32))
    return oracle.stack_scores(inp, mode="mirror", return_hidden=True)["h_final"][0]


def _layer_weights(H, rng, wq=0.0, wk=0.0, wv=1.0 / 3.0, wkc=0.0, wvc=1.0 / 3.0, wo=0.75):
    eye = np.eye(H)
    return dict(Wq=wq * eye, Wk=wk * eye, Wv=wv * eye, Wkc=wkc * eye, Wvc=wvc * eye, Wo=wo * eye)


def _h0(rng, Lq, H):
    return rng.standard_normal((Lq, H)).astype(np.float32).astype(np.float64)   # not bf16-representable


def test_mirror_one_visible_key_rounds_the_layer_input_and_keeps_fp32_residual():
    # one position, empty passage: the output is the single value row
    # V = bf16(bf16(h) Wv^T); the residual is stored in fp32
    rng = np.random.default_rng(31)
    H = 64
    h0 = _h0(rng, 1, H)
    W = _layer_weights(H, rng, wq=0.5, wk=0.25)
    x = np.full((4, H), np.nan)
    got = _one_pair(h0, x, np.zeros(4), W)
    V = _bf(_bf(h0) / 3.0)
    np.testing.assert_array_equal(got, _f32(h0 + V * 0.75)[-1])


def test_mirror_uniform_weights_round_values_and_output():
    # Wq = 0: every logit is 0, so row 1's output is bf16((V0 + V1) / 2)
    rng = np.random.default_rng(32)
    H, Lq = 64, 2
    h0 = _h0(rng, Lq, H)
    W = _layer_weights(H, rng, wk=0.5)
    got = _one_pair(h0, np.full((4, H), np.nan), np.zeros(4), W)
    V = _bf(_bf(h0) / 3.0)
    O1 = _bf((V[0] + V[1]) / 2)
    np.testing.assert_array_equal(got, _f32(h0[1] + O1 * 0.75))


def test_mirror_two_keys_round_queries_and_keys():
    # row 1 of two positions: weights sigma(s1 - s0), sigma(s0 - s1) with
    # s_j = bf16(0.3 bf16(h1)) . bf16(0.7 bf16(h_j)) / sqrt(d)
    rng = np.random.default_rng(33)
    H, Lq = 64, 2
    h0 = _h0(rng, Lq, H) * 0.5
    W = _layer_weights(H, rng, wq=0.3, wk=0.7)
    got = _one_pair(h0, np.full((4, H), np.nan), np.zeros(4), W)
    hb = _bf(h0)
    q1, K, V = _bf(0.3 * hb[1]), _bf(0.7 * hb), _bf(hb / 3.0)
    s = (K @ q1) / math.sqrt(H)
    p1 = 1.0 / (1.0 + math.exp(s[0] - s[1]))
    O1 = _bf((1.0 - p1) * V[0] + p1 * V[1])
    np.testing.assert_allclose(got, _f32(h0[1] + O1 * 0.75), rtol=0, atol=1e-12)


def test_mirror_cross_chunk_rounds_pooled_and_cross_values():
    # one position, a passage of 3 valid tokens in one chunk, Wq = 0: the
    # output is bf16((V0 + Vc) / 2), Vc = bf16(bf16(mean of the tokens) / 3)
    rng = np.random.default_rng(34)
    H = 64
    h0 = _h0(rng, 1, H)
    x = rng.standard_normal((4, H)).astype(np.float32).astype(np.float64)
    mask = np.array([1, 1, 1, 0])
    x[3] = np.nan
    W = _layer_weights(H, rng, wk=0.5, wkc=0.5)
    got = _one_pair(h0, x, mask, W)
    V0 = _bf(_bf(h0[0]) / 3.0)
    Vc = _bf(_bf(x[:3].mean(axis=0)) / 3.0)
    np.testing.assert_array_equal(got, _f32(h0[0] + _bf((V0 + Vc) / 2) * 0.75))


def test_mirror_cross_chunk_key_rounding():
    # one position and one chunk with a real query: the logistic weight of
    # the cross key uses kc = bf16(0.9 bf16(pooled))
    rng = np.random.default_rng(35)
    H = 64
    h0 = _h0(rng, 1, H) * 0.5
    x = rng.standard_normal((4, H)).astype(np.float32).astype(np.float64)
    mask = np.array([1, 1, 0, 0])
    x[2:] = np.nan
    W = _layer_weights(H, rng, wq=0.3, wk=0.7, wkc=0.9)
    got = _one_pair(h0, x, mask, W)
    hb = _bf(h0[0])
    pooled = _bf(x[:2].mean(axis=0))
    q, k0, kc = _bf(0.3 * hb), _bf(0.7 * hb), _bf(0.9 * pooled)
    V0, Vc = _bf(hb / 3.0), _bf(pooled / 3.0)
    pc = 1.0 / (1.0 + math.exp((q @ k0 - q @ kc) / math.sqrt(H)))
    O = _bf((1.0 - pc) * V0 + pc * Vc)
    np.testing.assert_allclose(got, _f32(h0[0] + O * 0.75), rtol=0, atol=1e-12)


# ------------------------------------------------------------------ stack
def _tiny_inputs(n_layers=2, seed=5, shape=None):
    return synth.make_inputs(0, seed=seed, n_layers=n_layers, shape=shape)


def test_stack_zero_wo_is_identity_closed_form():
    inp = _tiny_inputs(n_layers=3)
    for W in inp["layers"]:
        W["Wo"] = np.zeros_like(W["Wo"])
    res = oracle.stack_scores(inp, mode="pure")
    sh = inp["shape"]
    lq = inp["lq"]
    h_last = inp["h0"][lq[0] - 1].astype(np.float64)
    w = inp["w_yesno"].astype(np.float64)
    margin = h_last @ (w[0] - w[1])
    np.testing.assert_allclose(res["margin"], np.full(sh.pairs, margin), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(res["score"], scipy.special.expit(margin), rtol=1e-12)


def test_stack_identical_docs_identical_scores_and_order_independence():
    inp = _tiny_inputs(n_layers=2)
    inp["x"][3] = inp["x"][1]
    inp["token_mask"][3] = inp["token_mask"][1]
    res = oracle.stack_scores(inp, mode="pure")
    assert res["score"][3] == res["score"][1]
    sub = oracle.stack_scores(inp, pairs=[6, 2, 4], mode="pure")
    np.testing.assert_array_equal(sub["score"], res["score"][[6, 2, 4]])


def _torch_stack_one_pair(h0, x_doc, mask_doc, layers, w_yesno, nq, nkv, d):
    """Independent fp64 formulation of the same layer reading with torch:
    pooling by reshaping into groups of 4 and dividing by the valid counts,
    SDPA over the concatenated KV with a boolean mask."""
    T, H = x_doc.shape
    Tp = -(-T // 4) * 4
    xs = torch.zeros(Tp, H, dtype=torch.float64)
    ms = torch.zeros(Tp, dtype=torch.float64)
    m = torch.as_tensor(mask_doc, dtype=torch.float64)
    xs[:T] = torch.where(m[:, None] > 0, torch.as_tensor(np.nan_to_num(x_doc), dtype=torch.float64), 0.0)
    ms[:T] = m
    cnt = ms.view(-1, 4).sum(1)
    pooled = xs.view(-1, 4, H).sum(1) / cnt.clamp(min=1)[:, None]
    cvalid = cnt > 0
    h = torch.as_tensor(h0, dtype=torch.float64)
    Lq = h.shape[0]
    for W in layers:
        t = {k: torch.as_tensor(v, dtype=torch.float64) for k, v in W.items()}
        q = (h @ t["Wq"].T).view(Lq, nq, d)
        k = torch.cat([(h @ t["Wk"].T).view(Lq, nkv, d), (pooled @ t["Wkc"].T).view(-1, nkv, d)], 0)
        v = torch.cat([(h @ t["Wv"].T).view(Lq, nkv, d), (pooled @ t["Wvc"].T).view(-1, nkv, d)], 0)
        k = k.repeat_interleave(nq // nkv, 1).transpose(0, 1)
        v = v.repeat_interleave(nq // nkv, 1).transpose(0, 1)
        allow = torch.cat([torch.ones(Lq, Lq, dtype=torch.bool).tril(), cvalid[None].expand(Lq, -1)], 1)
        o = torch.nn.functional.scaled_dot_product_attention(q.transpose(0, 1), k, v, attn_mask=allow)
        h = h + o.transpose(0, 1).reshape(Lq, nq * d) @ t["Wo"].T
    w = torch.as_tensor(w_yesno, dtype=torch.float64)
    margin = float(h[-1] @ (w[0] - w[1]))
    return margin


def test_stack_pure_matches_independent_torch_formulation():
    inp = _tiny_inputs(n_layers=2, seed=17)
    sh = inp["shape"]
    res = oracle.stack_scores(inp, mode="pure")
    for p in range(sh.pairs):
        dd = p % sh.n_docs
        m = _torch_stack_one_pair(inp["h0"], inp["x"][dd], inp["token_mask"][dd], inp["layers"], inp["w_yesno"],
                                  sh.nq, sh.nkv, sh.d)
        assert math.isclose(res["margin"][p], m, rel_tol=1e-10, abs_tol=1e-12)


def test_stack_mirror_close_to_pure_on_bf16_shape():
    # rounding to bf16 at the storage points moves scores by far less than the
    # 5e-3 score tolerance (noise floor of the bf16 storage itself)
    sh = synth.Shape("mini_bf16", 2, 4, 64, 128, 4, 1, 32, 3, "bf16", ("loguniform", 8, 64), ("uniform", 5, 20))
    inp = synth.make_inputs(0, seed=3, shape=sh)
    pure = oracle.stack_scores(inp, mode="pure")
    mirror = oracle.stack_scores(inp, mode="mirror")
    d = np.abs(pure["score"] - mirror["score"])
    assert d.max() < 5e-3 and d.max() > 0


# ------------------------------------------------------------------ model-shaped layer parts
def test_rms_norm_worked_example_library_and_scale_invariance():
    y = oracle.rms_norm(np.array([[3.0, 4.0]]), np.array([1.0, 2.0]), eps=0.0)
    r = math.sqrt((9 + 16) / 2)
    np.testing.assert_allclose(y, [[3 / r, 8 / r]], rtol=1e-15)
    rng = np.random.default_rng(4)
    x = rng.standard_normal((7, 48))
    w = 1 + 0.1 * rng.standard_normal(48)
    ref = torch.nn.functional.rms_norm(torch.as_tensor(x), (48,), torch.as_tensor(w), eps=1e-6).numpy()
    np.testing.assert_allclose(oracle.rms_norm(x, w, 1e-6), ref, rtol=1e-12, atol=1e-14)
    # without eps the output ignores the row's scale, and with unit weight its mean square is 1
    np.testing.assert_allclose(oracle.rms_norm(5 * x, w, 0.0), oracle.rms_norm(x, w, 0.0), rtol=1e-13)
    np.testing.assert_allclose(np.mean(oracle.rms_norm(x, np.ones(48), 0.0) ** 2, axis=1), 1.0, rtol=1e-13)


def test_rope_pairing_frequencies_and_relative_position():
    # rotate-half pairing: dim 0 turns with dim d/2 = 2 at frequency theta^0 = 1,
    # dim 1 with dim 3 at theta^(-2/4) = 0.01 (theta = 10^4)
    e0 = oracle.rope(np.array([[[1.0, 0.0, 0.0, 0.0]]]), [1], 1e4)[0, 0]
    np.testing.assert_allclose(e0, [math.cos(1), 0, math.sin(1), 0], atol=1e-15)
    e1 = oracle.rope(np.array([[[0.0, 1.0, 0.0, 0.0]]]), [1], 1e4)[0, 0]
    np.testing.assert_allclose(e1, [0, math.cos(0.01), 0, math.sin(0.01)], atol=1e-15)
    rng = np.random.default_rng(8)
    q = rng.standard_normal((1, 3, 16))
    k = rng.standard_normal((1, 3, 16))
    # position 0 is the identity; every rotation keeps the norm
    np.testing.assert_array_equal(oracle.rope(q, [0], 500.0), q)
    np.testing.assert_allclose(np.linalg.norm(oracle.rope(q, [37], 500.0), axis=-1), np.linalg.norm(q, axis=-1),
                               rtol=1e-13)
    # the score of a rotated query and key depends on the positions only through their difference
    for m, n in [(5, 2), (40, 33), (7, 7), (3, 9)]:
        a = np.sum(oracle.rope(q, [m], 500.0) * oracle.rope(k, [n], 500.0), axis=-1)
        b = np.sum(oracle.rope(q, [m - n], 500.0) * k, axis=-1)
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)
    # the same rotation written as complex multiplication of (x_i + i x_{i+d/2})
    pos = np.array([0, 1, 4, 11])
    x = rng.standard_normal((4, 2, 8))
    z = torch.complex(torch.as_tensor(x[..., :4]), torch.as_tensor(x[..., 4:]))
    ang = torch.as_tensor(pos, dtype=torch.float64)[:, None] * (1e4 ** (-torch.arange(0, 8, 2, dtype=torch.float64)
                                                                        / 8))[None]
    zr = z * torch.polar(torch.ones_like(ang), ang)[:, None, :]
    ref = torch.cat([zr.real, zr.imag], -1).numpy()
    np.testing.assert_allclose(oracle.rope(x, pos, 1e4), ref, rtol=1e-12, atol=1e-14)


def test_gelu_tanh_library_odd_identity_and_exact_gelu():
    x = np.linspace(-8, 8, 2001)
    ref = torch.nn.functional.gelu(torch.as_tensor(x), approximate="tanh").numpy()
    np.testing.assert_allclose(oracle.gelu_tanh(x), ref, rtol=1e-12, atol=1e-15)
    # gelu(x) - gelu(-x) = x holds exactly for the tanh form
    np.testing.assert_allclose(oracle.gelu_tanh(x) - oracle.gelu_tanh(-x), x, atol=1e-13)
    # and it stays within 1e-3 of the exact x * Phi(x)
    exact = x * 0.5 * (1 + scipy.special.erf(x / math.sqrt(2)))
    assert np.max(np.abs(oracle.gelu_tanh(x) - exact)) < 1e-3
    np.testing.assert_allclose(oracle.gated_gelu(x, 3.0), 3.0 * ref, rtol=1e-12, atol=1e-14)


def _model_inputs(n_layers=2, seed=21, mlp_dim=48):
    sh = synth.Shape("mini_model_f32", 1, 3, 16, 32, 4, 2, 8, n_layers, "f32", ("loguniform", 4, 16),
                     ("const", 6, 6))
    return synth.make_inputs(0, seed=seed, shape=sh, mlp_dim=mlp_dim)


def _torch_model_stack_one_pair(h0, x_doc, mask_doc, layers, model, w_yesno, nq, nkv, d):
    """Independent fp64 formulation of the model-shaped layer with torch
    library routines: rms_norm, complex-multiplication RoPE, SDPA over the
    concatenated KV, tanh-GELU."""
    F = torch.nn.functional
    T, H = x_doc.shape
    m = torch.as_tensor(mask_doc, dtype=torch.float64)
    xs = torch.where(m[:, None] > 0, torch.as_tensor(np.nan_to_num(x_doc), dtype=torch.float64), 0.0)
    cnt = m.view(-1, 4).sum(1)
    pooled = xs.view(-1, 4, H).sum(1) / cnt.clamp(min=1)[:, None]
    cvalid = cnt > 0
    h = torch.as_tensor(h0, dtype=torch.float64)
    Lq = h.shape[0]
    eps = model["eps"]
    ang = torch.arange(Lq, dtype=torch.float64)[:, None] * (
        model["rope_theta"] ** (-torch.arange(0, d, 2, dtype=torch.float64) / d))[None]
    rot = torch.polar(torch.ones_like(ang), ang)[:, None, :]

    def rope(t):
        z = torch.complex(t[..., : d // 2], t[..., d // 2:]) * rot
        return torch.cat([z.real, z.imag], -1)

    for W in layers:
        t = {k: torch.as_tensor(v, dtype=torch.float64) for k, v in W.items()}
        x = F.rms_norm(h, (H,), t["attn_norm"], eps=eps)
        q = rope((x @ t["Wq"].T).view(Lq, nq, d))
        ks = rope((x @ t["Wk"].T).view(Lq, nkv, d))
        k = torch.cat([ks, (pooled @ t["Wkc"].T).view(-1, nkv, d)], 0)
        v = torch.cat([(x @ t["Wv"].T).view(Lq, nkv, d), (pooled @ t["Wvc"].T).view(-1, nkv, d)], 0)
        k = k.repeat_interleave(nq // nkv, 1).transpose(0, 1)
        v = v.repeat_interleave(nq // nkv, 1).transpose(0, 1)
        allow = torch.cat([torch.ones(Lq, Lq, dtype=torch.bool).tril(), cvalid[None].expand(Lq, -1)], 1)
        o = F.scaled_dot_product_attention(q.transpose(0, 1), k, v, attn_mask=allow)
        h = h + o.transpose(0, 1).reshape(Lq, nq * d) @ t["Wo"].T
        x2 = F.rms_norm(h, (H,), t["mlp_norm"], eps=eps)
        h = h + (F.gelu(x2 @ t["Wg"].T, approximate="tanh") * (x2 @ t["Wu"].T)) @ t["Wd"].T
    last = F.rms_norm(h[-1], (H,), torch.as_tensor(model["final_norm"], dtype=torch.float64), eps=eps)
    w = torch.as_tensor(w_yesno, dtype=torch.float64)
    return float(last @ (w[0] - w[1]))


def test_model_stack_pure_matches_independent_torch_formulation():
    inp = _model_inputs()
    sh = inp["shape"]
    res = oracle.stack_scores(inp, mode="pure")
    for p in range(sh.pairs):
        dd = p % sh.n_docs
        mg = _torch_model_stack_one_pair(inp["h0"], inp["x"][dd], inp["token_mask"][dd], inp["layers"],
                                         inp["model"], inp["w_yesno"], sh.nq, sh.nkv, sh.d)
        assert math.isclose(res["margin"][p], mg, rel_tol=1e-10, abs_tol=1e-12)


def test_model_layer_reduces_to_plain_layer():
    # one decoder position (RoPE at position 0 is the identity), unit-rms input,
    # unit norm weights, no eps, a zero down projection and no final norm: the
    # model-shaped layer is the plain one
    inp = _model_inputs(n_layers=1, seed=5)
    sh = dataclasses.replace(inp["shape"], lq=("const", 1, 1))
    inp = synth.make_inputs(0, seed=5, shape=sh, mlp_dim=48)
    h0 = inp["h0"].astype(np.float64)
    inp["h0"] = h0 / np.sqrt(np.mean(h0 * h0, axis=1, keepdims=True))
    for W in inp["layers"]:
        W["attn_norm"] = np.ones_like(W["attn_norm"])
        W["Wd"] = np.zeros_like(W["Wd"])
    model = dict(inp["model"], eps=0.0, final_norm=None)
    plain = oracle.stack_scores(dict(inp, model=None), mode="pure")
    shaped = oracle.stack_scores(dict(inp, model=model), mode="pure")
    np.testing.assert_allclose(shaped["margin"], plain["margin"], rtol=1e-12, atol=1e-14)


# ------------------------------------------------------------------ ranking
def test_rank_worked_example():
    ex = json.load(open(os.path.join(GOLD, "rank_worked_example.json")))
    sc = np.array([[np.nan if v is None else v for v in row] for row in ex["scores"]])
    idx, val = oracle.rank_topn(sc, ex["top_n"])
    assert idx.tolist() == ex["index"]
    assert np.array_equal(val, np.array(ex["relevance_score"]))


def test_rank_is_a_stable_descending_permutation():
    rng = np.random.default_rng(5)
    sc = np.round(rng.random((7, 50)) * 8) / 8          # many ties
    sc[2, [3, 9, 10]] = np.nan
    idx, val = oracle.rank_topn(sc, 50)
    for q in range(7):
        assert sorted(idx[q].tolist()) == list(range(50))   # a permutation
        finite = ~np.isnan(val[q])
        assert np.all(np.diff(val[q][finite]) <= 0)         # non-increasing
        assert not np.any(finite[np.argmin(finite):]) or finite.all()  # NaNs only at the end
        for a in range(49):                                  # ties by index
            if val[q, a] == val[q, a + 1] or (np.isnan(val[q, a]) and np.isnan(val[q, a + 1])):
                assert idx[q, a] < idx[q, a + 1]
    # numpy's stable argsort of the negated scores agrees where no NaN is present
    ref = np.argsort(-sc[0], kind="stable")
    assert np.array_equal(idx[0], ref)

