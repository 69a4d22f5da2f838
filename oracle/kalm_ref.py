"""Plain fp64 definitions of the KaLM-Reranker-V1 hot path (CPU oracle).

TEST INFRASTRUCTURE ONLY: imported by tests, by ``__graft_entry__.smoke()``
and by the CPU-baseline leg of ``bench.py``; never by the product path.

Sources (web pages; cited by title and section):
  [MLX]   "KaLM-Reranker-V1-Nano -- MLX (Apple Silicon)", sections
          "What this is" (the three-step relevance pipeline) and "Speed"
          (encodings computed once and reused across queries).
  [Q4KM]  "KaLM-Reranker-V1-Small Q4_K_M GGUF", sections "Score a pair"
          (score = sigmoid(yes_logit - no_logit)) and "Runtime boundaries"
          (encoder limit 1024 tokens, query budget 512, chunk size 4).
  [Q80]   "KaLM-Reranker-V1-Large Q8_0 GGUF", section "Frozen inference
          contract" (right padding, masked mean over consecutive groups of 4
          tokens, yes/no token rows, score = sigmoid of the margin).
  [PAPER] "KaLM-Reranker-V1: Fast but Not Late Interaction for Compressed
          Document Reranking", abstract (encoder pre-encodes passages with
          Matryoshka pooling; decoder cross-attends to them).
  The optional model-shaped layer parts (rms_norm, rope, gelu_tanh,
  gated_gelu) follow [MLX] "What this is" / "Derivation" (every dim and RoPE
  parameter read from the config, RoPE inverse frequencies computed from it)
  in their standard forms, each marked READING.

Every function computes in float64 on the exact values it is handed.  Where a
page leaves a step open the plainest reading is taken; each such reading is
marked READING below.

Rounding mirrors: the ``mirror`` stack mode rounds to the storage type at the
points where the HIP path stores a tensor (bf16 or fp32), so the two can be
compared layer after layer; ``pure`` mode never rounds.  ``round_bf16`` is
written from the definition of the format: keep 8 significant bits, ties to
even.

Parity unpinned: none (see tests/test_oracle.py for the pin of every function).
"""
from __future__ import annotations

import math
from typing import Callable, Dict, Iterable, List, Optional, Sequence

import numpy as np

F64 = np.float64


# --------------------------------------------------------------------------
# storage rounding (used only by the mirror mode)
# --------------------------------------------------------------------------
def round_bf16(a) -> np.ndarray:
    """Nearest bf16 value (ties to even), as float64.

    bf16 has float32's sign and 8-bit exponent and 7 stored significand
    bits.  A value in [2^(e-1), 2^e) at or above 2^-126 keeps 8 significant
    bits (its quantum is 2^(e-8)); below 2^-126 the representable values are
    the multiples of 2^-133 (subnormals); a value that rounds to 2^128 or
    beyond is +-inf.  Rounding to a multiple of the quantum with ties to even
    is ties-to-even on the stored significand.  NaN stays NaN.
    """
    a = np.asarray(a, dtype=F64)
    _, e = np.frexp(a)                          # |a| in [2^(e-1), 2^e)
    q = np.maximum(e - 8, -133)                 # exponent of the quantum
    r = np.ldexp(np.rint(np.ldexp(a, -q)), q)   # np.rint rounds half to even
    return np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, a), r)


def round_f32(a) -> np.ndarray:
    """Nearest float32 value (IEEE round to nearest even), as float64."""
    return np.asarray(a, dtype=F64).astype(np.float32).astype(F64)


def _identity(a):
    return np.asarray(a, dtype=F64)


# --------------------------------------------------------------------------
# a1: chunk pooling
# --------------------------------------------------------------------------
def chunk_pool(x, token_mask, chunk: int = 4):
    """Masked mean over consecutive groups of ``chunk`` encoder tokens.

    [Q80] Frozen inference contract: encoder states are mean-pooled, under the
    padding mask, over consecutive groups of 4 tokens; [MLX] What this is:
    chunk size 4, masked mean per chunk, giving the cached document vectors.

    READING: chunk c covers tokens [c*chunk, (c+1)*chunk) counted from token 0
    of the right-padded sequence; the mean divides by the number of valid
    tokens in the chunk (a partial last chunk averages only its valid tokens);
    a chunk without valid tokens is 0 with chunk_mask 0; arbitrary 0/1 masks
    are allowed (right padding is the case the pages use).

    x [D,T,H], token_mask [D,T] -> pooled [D,C,H] float64, chunk_mask [D,C]
    uint8, n_chunks [D] int32, with C = ceil(T / chunk).
    """
    x = np.asarray(x)
    token_mask = np.asarray(token_mask)
    D, T, H = x.shape
    C = -(-T // chunk) if T > 0 else 0
    pooled = np.zeros((D, C, H), dtype=F64)
    cmask = np.zeros((D, C), dtype=np.uint8)
    for d in range(D):
        for c in range(C):
            t0, t1 = c * chunk, min(T, (c + 1) * chunk)
            valid = token_mask[d, t0:t1] != 0
            cnt = int(valid.sum())
            if cnt > 0:
                rows = x[d, t0:t1][valid].astype(F64)
                pooled[d, c] = rows.sum(axis=0) / cnt
                cmask[d, c] = 1
    n_chunks = cmask.sum(axis=1).astype(np.int32)
    return pooled, cmask, n_chunks


# --------------------------------------------------------------------------
# a2: cross K/V projection
# --------------------------------------------------------------------------
def cross_kv(pooled, Wk, Wv):
    """Cross-attention keys and values of the cached pooled passage vectors.

    [MLX] What this is: the decoder's cross-attention K/V are computed over
    the cached passage encodings.  READING: a plain bias-free linear map with
    weights in [out, in] layout, K = pooled @ Wk^T and V = pooled @ Wv^T.

    pooled [..., H], Wk/Wv [nkv*d, H] -> Kc, Vc [..., nkv*d] float64.
    """
    p = np.asarray(pooled, dtype=F64)
    return p @ np.asarray(Wk, dtype=F64).T, p @ np.asarray(Wv, dtype=F64).T


# --------------------------------------------------------------------------
# a3: merged self + cross attention (one pair)
# --------------------------------------------------------------------------
def merged_attn(Q, Ks, Vs, Kc, Vc, chunk_mask, scale: Optional[float] = None):
    """One softmax over the concatenation [causal self keys ; valid cross keys].

    [MLX] What this is: a single fused scaled-dot-product attention whose KV is
    the decoder's self-attention KV concatenated with cross-attention KV of the
    cached passage.  Written as the definition: the explicit concatenated
    logit row, a two-pass softmax (max, then normalised exponentials), and the
    probability-weighted sum of the concatenated values.

    READINGS: scale = 1/sqrt(d) unless given; decoder row i sees self keys
    j <= i; cross chunk c is visible iff chunk_mask[c] != 0; query head h
    reads KV head h // (nq // nkv); no softcap, bias or window.

    Q [Lq,nq,d], Ks/Vs [Lq,nkv,d], Kc/Vc [C,nkv,d], chunk_mask [C]
    -> O [Lq,nq,d] float64, lse [Lq,nq] float64 (natural-log log-sum-exp of
    the scaled logits).
    """
    Q = np.asarray(Q, dtype=F64)
    Ks = np.asarray(Ks, dtype=F64)
    Vs = np.asarray(Vs, dtype=F64)
    Lq, nq, d = Q.shape
    nkv = Ks.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    valid = np.nonzero(np.asarray(chunk_mask) != 0)[0]
    Kc = np.asarray(Kc, dtype=F64)[valid]
    Vc = np.asarray(Vc, dtype=F64)[valid]
    group = nq // nkv
    causal = np.tril(np.ones((Lq, Lq), dtype=bool))
    O = np.zeros((Lq, nq, d), dtype=F64)
    lse = np.zeros((Lq, nq), dtype=F64)
    for h in range(nq):
        g = h // group
        s_self = (Q[:, h] @ Ks[:, g].T) * scale
        s_self = np.where(causal, s_self, -np.inf)
        s_cross = (Q[:, h] @ Kc[:, g].T) * scale
        s = np.concatenate([s_self, s_cross], axis=1)
        v = np.concatenate([Vs[:, g], Vc[:, g]], axis=0)
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        tot = e.sum(axis=1, keepdims=True)
        O[:, h] = (e / tot) @ v
        lse[:, h] = (m + np.log(tot))[:, 0]
    return O, lse


def merged_attn_partial(Q, K, V, allowed, scale: float):
    """Softmax attention of Q [Lq,d] over an explicit key set K/V [n,d] with a
    boolean visibility matrix ``allowed`` [Lq,n]; returns (O, lse).  Rows with
    no visible key give O = 0 and lse = -inf.  Used to state the split of the
    merged softmax into a self part and a cross part."""
    Q = np.asarray(Q, dtype=F64)
    K = np.asarray(K, dtype=F64)
    V = np.asarray(V, dtype=F64)
    s = np.where(allowed, (Q @ K.T) * scale, -np.inf)
    Lq = Q.shape[0]
    O = np.zeros((Lq, V.shape[1]), dtype=F64)
    lse = np.full(Lq, -np.inf)
    for i in range(Lq):
        if not allowed[i].any():
            continue
        m = s[i][allowed[i]].max()
        e = np.where(allowed[i], np.exp(s[i] - m), 0.0)
        tot = e.sum()
        O[i] = (e / tot) @ V
        lse[i] = m + math.log(tot)
    return O, lse


# --------------------------------------------------------------------------
# a4: yes/no readout
# --------------------------------------------------------------------------
def yesno_score(h_final, w_yesno):
    """Relevance score from the decoder's final hidden state.

    [MLX] What this is: score = softmax([logit_yes, logit_no])[yes] read at
    the final decoder position.  [Q4KM] Score a pair / [Q80] Frozen inference
    contract: margin = yes_logit - no_logit and score = sigmoid(margin); rank
    by the margin.  READING: the two logits are dot products of the final
    hidden state with the two LM-head rows (row 0 = "yes", row 1 = "no"); no
    final norm or softcap.

    h_final [..., H], w_yesno [2, H] -> dict(yes, no, margin, score, softmax2)
    where ``score`` uses the overflow-free sigmoid form and ``softmax2`` the
    explicit two-way softmax (the two are equal).
    """
    h = np.asarray(h_final, dtype=F64)
    w = np.asarray(w_yesno, dtype=F64)
    y = h @ w[0]
    n = h @ w[1]
    m = y - n
    pos = m >= 0
    e = np.exp(-np.abs(m))
    score = np.where(pos, 1.0 / (1.0 + e), e / (1.0 + e))
    top = np.maximum(y, n)
    ey, en = np.exp(y - top), np.exp(n - top)
    return dict(yes=y, no=n, margin=m, score=score, softmax2=ey / (ey + en))


# --------------------------------------------------------------------------
# ranking of a query's passages (the step above the score)
# --------------------------------------------------------------------------
def rank_topn(scores, top_n: int):
    """Top-n passages of each query, best first.

    [MLX] What this is / Files: rerank(query, docs, top_n) returns the passages
    highest relevance score first as (index, relevance_score); [Q4KM] Score a
    pair: rank larger margins first (the score is increasing in the margin).
    READING: equal scores keep input order (lower index first); NaN scores
    (a pair with no valid score) go last, by index.

    scores [Q, D] -> (index [Q, top_n] int, score [Q, top_n])
    """
    s = np.asarray(scores, dtype=F64)
    Qn, D = s.shape
    idx = np.zeros((Qn, top_n), dtype=np.int64)
    val = np.zeros((Qn, top_n), dtype=F64)
    for q in range(Qn):
        order = sorted(range(D), key=lambda j: (math.isnan(s[q, j]), 0.0 if math.isnan(s[q, j]) else -s[q, j], j))
        idx[q] = order[:top_n]
        val[q] = s[q, order[:top_n]]
    return idx, val


# --------------------------------------------------------------------------
# a0: ragged batch layout
# --------------------------------------------------------------------------
def pair_layout(lq: Sequence[int], n_docs: int):
    """Row layout of a batch in which every query is paired with every doc.

    READING: pair p joins query p // D with doc p % D (each query reranks the
    same D candidates, [MLX] Speed: the same document set reranked against
    many queries); pair p's decoder rows are packed one after another; the
    score is read at the pair's last row ([MLX] What this is: final position).

    Returns dict(cu_q [P+1], doc_of_pair [P], query_of_pair [P],
    final_row [P], h0_row [rows], h0_final [P], cu_u [Q+1]) as int32, where
    h0_row[r] is the row of the query's first-layer hidden state that pair row
    r starts from, h0_final[p] that row for the pair's final position, and
    cu_u the row offsets of the queries' own rows (packed in order).
    """
    lq = [int(v) for v in lq]
    Qn = len(lq)
    P = Qn * n_docs
    cu_q = [0]
    doc_of_pair, query_of_pair, final_row, h0_row, h0_final = [], [], [], [], []
    q_start = [0]
    for v in lq:
        q_start.append(q_start[-1] + v)
    for p in range(P):
        q, dd = p // n_docs, p % n_docs
        n = lq[q]
        doc_of_pair.append(dd)
        query_of_pair.append(q)
        final_row.append(cu_q[-1] + n - 1)
        h0_final.append(q_start[q] + n - 1)
        for r in range(n):
            h0_row.append(q_start[q] + r)
        cu_q.append(cu_q[-1] + n)
    i32 = lambda v: np.asarray(v, dtype=np.int32)
    return dict(cu_q=i32(cu_q), doc_of_pair=i32(doc_of_pair), query_of_pair=i32(query_of_pair),
                final_row=i32(final_row), h0_row=i32(h0_row), h0_final=i32(h0_final), cu_u=i32(q_start))


# --------------------------------------------------------------------------
# Decoder-layer completion (a model-shaped layer around a3)
# --------------------------------------------------------------------------
def rms_norm(x, w, eps: float = 1e-6):
    """Root-mean-square normalisation of each row, times a per-column weight.

    The pages name no norm; they say every dim and RoPE parameter comes from
    the model's config ([MLX] What this is).  READING: the standard form
    y = x / sqrt(mean(x^2) + eps) * w (a plain weight, eps from config,
    1e-6 by default).  x [..., H], w [H] -> float64.
    """
    x = np.asarray(x, dtype=F64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(w, dtype=F64)


def rope(x, positions, theta: float = 10000.0):
    """Rotary position embedding of x [L, n_heads, d] at ``positions`` [L].

    [MLX] Derivation: the inverse-frequency tables are computed from the
    config.  READING: inverse frequency theta^(-2i/d) for i < d/2, and the
    "rotate half" pairing -- dim i turns together with dim i + d/2 by the
    angle position * theta^(-2i/d).
    """
    x = np.asarray(x, dtype=F64)
    d = x.shape[-1]
    half = d // 2
    inv_freq = float(theta) ** (-2.0 * np.arange(half) / d)
    ang = np.asarray(positions, dtype=F64)[:, None] * inv_freq[None, :]   # [L, d/2]
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def gelu_tanh(x):
    """GELU in its tanh form, 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))).

    READING: the gated MLP's activation (the pages name none; the tanh form is
    the one used by the Gemma family that T5-Gemma builds on).
    """
    x = np.asarray(x, dtype=F64)
    return 0.5 * x * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (x + 0.044715 * x ** 3)))


def gated_gelu(g, u):
    """The gated MLP's activation: gelu_tanh(gate) * up, elementwise."""
    return gelu_tanh(g) * np.asarray(u, dtype=F64)


# --------------------------------------------------------------------------
# a5: the decoder stack glue (one pair)
# --------------------------------------------------------------------------
def _store_fn(mode: str, dtype: str) -> Callable:
    if mode == "pure":
        return _identity
    if mode != "mirror":
        raise ValueError(mode)
    return round_bf16 if dtype == "bf16" else round_f32


def decoder_stack(h0, pooled_doc, chunk_mask_doc, layers: List[Dict[str, np.ndarray]], w_yesno,
                  nq: int, nkv: int, d: int, mode: str = "mirror", dtype: str = "bf16",
                  return_hidden: bool = False, model: Optional[Dict[str, object]] = None):
    """Run one (query, passage) pair through the merged-attention stack.

    READING (the pages give only the layer counts and the merged attention
    itself, [MLX] What this is): each layer is
        hb = store(h);  Q, Ks, Vs = store(hb Wq^T), store(hb Wk^T), store(hb Wv^T)
        Kc, Vc = store(pooled Wkc^T), store(pooled Wvc^T)   (valid chunks only)
        O = store(merged_attn(Q, Ks, Vs, Kc, Vc))
        h = h + O Wo^T             (residual kept in fp32 storage)
    with no norm, RoPE or MLP; the score is read at the last row.  ``store``
    rounds to the storage dtype in mirror mode and is the identity in pure
    mode; h itself is rounded to fp32 after each layer in mirror mode.

    With ``model`` (dict rope_theta, eps, final_norm [H] or None) each layer
    is the model-shaped reading (pre-norm, RoPE on the self Q/K, gated MLP):
        hb = store(rms_norm(h, attn_norm))
        Q, Ks = store(rope(store(hb Wq^T))), store(rope(store(hb Wk^T)))  at
                positions 0..Lq-1; Vs, Kc, Vc as above (no RoPE on cross keys)
        h = h + store(merged_attn(...)) Wo^T
        x = store(rms_norm(h, mlp_norm))
        h = h + store(gated_gelu(store(x Wg^T), store(x Wu^T))) Wd^T
    and the score reads rms_norm(h_last, final_norm) when final_norm is given.

    h0 [Lq,H], pooled_doc [C,H] (already in storage precision), chunk_mask_doc
    [C] -> dict as ``yesno_score`` (+ ``h`` [Lq,H] when return_hidden).
    """
    st = _store_fn(mode, dtype)
    keep_f32 = round_f32 if mode == "mirror" else _identity
    h = np.asarray(h0, dtype=F64).copy()
    Lq = h.shape[0]
    pooled_doc = np.asarray(pooled_doc, dtype=F64)
    eps = float(model["eps"]) if model else 0.0
    for W in layers:
        hb = st(rms_norm(h, W["attn_norm"], eps)) if model else st(h)
        Qm = st(hb @ np.asarray(W["Wq"], F64).T).reshape(Lq, nq, d)
        Ks = st(hb @ np.asarray(W["Wk"], F64).T).reshape(Lq, nkv, d)
        Vs = st(hb @ np.asarray(W["Wv"], F64).T).reshape(Lq, nkv, d)
        if model:
            pos = np.arange(Lq)
            Qm = st(rope(Qm, pos, model["rope_theta"]))
            Ks = st(rope(Ks, pos, model["rope_theta"]))
        Kc, Vc = cross_kv(pooled_doc, W["Wkc"], W["Wvc"])
        Kc = st(Kc).reshape(-1, nkv, d)
        Vc = st(Vc).reshape(-1, nkv, d)
        O, _ = merged_attn(Qm, Ks, Vs, Kc, Vc, chunk_mask_doc)
        O = st(O).reshape(Lq, nq * d)
        h = keep_f32(h + O @ np.asarray(W["Wo"], F64).T)
        if model:
            x = st(rms_norm(h, W["mlp_norm"], eps))
            g = st(x @ np.asarray(W["Wg"], F64).T)
            u = st(x @ np.asarray(W["Wu"], F64).T)
            h = keep_f32(h + st(gated_gelu(g, u)) @ np.asarray(W["Wd"], F64).T)
    last = h[Lq - 1]
    if model and model.get("final_norm") is not None:
        last = keep_f32(rms_norm(last, model["final_norm"], eps))
    out = yesno_score(last, w_yesno)
    if return_hidden:
        out["h"] = h
    return out


def stack_scores(inputs: Dict[str, object], pairs: Optional[Iterable[int]] = None,
                 mode: str = "mirror", n_layers: Optional[int] = None, return_hidden: bool = False):
    """Score the pairs of a synthetic batch (all pairs by default).

    Pools every passage that a chosen pair needs (then rounds the pooled
    vectors to the storage dtype in mirror mode), and runs
    ``decoder_stack`` per pair.  Returns dict of float64 arrays yes, no,
    margin, score over the chosen pairs, plus ``pairs``; with
    ``return_hidden`` also ``h_final`` [pairs, H], each pair's hidden state
    at its final position after the last layer (before any final norm).
    """
    sh = inputs["shape"]
    D = sh.n_docs
    lq = np.asarray(inputs["lq"])
    q_start = np.concatenate([[0], np.cumsum(lq)])
    layers = inputs["layers"] if n_layers is None else inputs["layers"][:n_layers]
    pairs = list(range(sh.pairs)) if pairs is None else [int(p) for p in pairs]
    st = _store_fn(mode, sh.dtype)
    pooled_cache: Dict[int, tuple] = {}
    res = {k: [] for k in ("yes", "no", "margin", "score")}
    h_final = []
    for p in pairs:
        q, dd = p // D, p % D
        if dd not in pooled_cache:
            pooled, cm, _ = chunk_pool(inputs["x"][dd:dd + 1], inputs["token_mask"][dd:dd + 1], sh.chunk)
            pooled_cache[dd] = (st(pooled[0]), cm[0])
        pooled_doc, cm_doc = pooled_cache[dd]
        h0 = inputs["h0"][q_start[q]:q_start[q + 1]]
        out = decoder_stack(h0, pooled_doc, cm_doc, layers, inputs["w_yesno"],
                            sh.nq, sh.nkv, sh.d, mode=mode, dtype=sh.dtype, return_hidden=return_hidden,
                            model=inputs.get("model"))
        for k in res:
            res[k].append(float(out[k]))
        if return_hidden:
            h_final.append(out["h"][-1])
    res = {k: np.asarray(v, dtype=F64) for k, v in res.items()}
    res["pairs"] = np.asarray(pairs, dtype=np.int64)
    if return_hidden:
        res["h_final"] = np.asarray(h_final, dtype=F64).reshape(len(pairs), inputs["shape"].H)
    return res
