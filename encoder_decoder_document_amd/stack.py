"""Device-resident batch and the end-to-end hot-path step.

``upload`` copies a synthetic batch into HBM once (weights stacked the way the
kernels read them) and allocates every buffer the step writes, so the step
itself only enqueues libkalm calls on the current stream:

  kalm_pair_layout -> kalm_chunk_pool -> kalm_cross_kv_layers (every layer's cross
  K/V in one launch, shared by every query) -> kalm_gather_rows (each pair's residual stream starts from its
  query's first hidden state) -> per layer: kalm_linear (fused Q/K/V), kalm_merged_attn,
  kalm_linear (output projection added to the fp32 residual, bf16 copy for the
  next layer) -> kalm_yesno_score.  With ``prune`` the residual start is fused
  into the first layer's output projection (kalm_linear_residual adds it to the
  gathered first hidden states).

With ``prune`` (the default) two layers do less work for the same result:
  * layer 1: every passage of a query still holds the query's own first hidden
    states, so Q/K/V are projected once per query row (not once per pair row);
    the query's causal self-attention is computed once as well
    (kalm_self_attn_partial) and each pair is finished from it with its
    passage's cross keys (kalm_merged_attn_resume, shared rows) -- or, without
    ``reuse_self``, each pair reads the shared rows in one merged pass
    (kalm_merged_attn_rows, shared rows);
  * the last layer: the score reads only each pair's final position
    ("KaLM-Reranker-V1-Nano -- MLX (Apple Silicon)", What this is), so self K/V
    are projected for every row but Q, attention, the output projection and the
    residual update only for the final rows (kalm_merged_attn_rows, final row);
    in a one-layer stack, where the first layer is also the last, only the
    queries' own rows and each pair's final row are computed at all (shared
    final row; the residual starts from the query's final hidden state); with
    ``split_kv`` each pair's cross keys run in shares over several workgroups
    (kalm_merged_attn_split).

The decoder layer is the reading stated on the pages' behalf: the pages give
only the layer counts ("KaLM-Reranker-V1-Nano -- MLX (Apple Silicon)", What
this is) and the merged attention; no norm, RoPE or MLP is added.
"""
from __future__ import annotations

import contextlib
import dataclasses
import math
from typing import Dict, List, Optional

import numpy as np
import torch

from . import ops


@dataclasses.dataclass
class DeviceBatch:
    shape: object
    n_layers: int
    dtype: torch.dtype
    D: int
    T: int
    H: int
    nq: int
    nkv: int
    d: int
    chunk: int
    Cmax: int
    n_queries: int
    P: int
    rows: int
    max_lq: int
    # inputs
    x: torch.Tensor
    token_mask: torch.Tensor
    lq: torch.Tensor
    h0: torch.Tensor
    Wqkv: List[torch.Tensor]
    Wkvc: torch.Tensor          # [L, 2*kv, H]: every layer's cross K/V weights
    Wo: List[torch.Tensor]
    w_yesno: torch.Tensor
    # buffers written by the step
    buf: Dict[str, torch.Tensor]
    # model-shaped layer (RMSNorm, RoPE, gated MLP), when the batch carries its weights
    model: Optional[Dict[str, object]] = None


def upload(inputs: Dict[str, object], device="cuda", n_layers: Optional[int] = None) -> DeviceBatch:
    sh = inputs["shape"]
    dt = torch.bfloat16 if sh.dtype == "bf16" else torch.float32
    layers = inputs["layers"] if n_layers is None else inputs["layers"][:n_layers]
    L = len(layers)
    D, T, H = sh.n_docs, sh.T, sh.H
    chunk = sh.chunk
    Cmax = -(-T // chunk)
    lq = np.asarray(inputs["lq"], dtype=np.int32)
    P = sh.n_queries * D
    rows = int(D * lq.sum())
    kv = sh.nkv * sh.d
    nqkv = sh.nq * sh.d + 2 * kv

    def dev(a, dtype=dt):
        return torch.from_numpy(np.ascontiguousarray(a)).to(device=device, dtype=dtype)

    Wqkv = [dev(np.concatenate([W["Wq"], W["Wk"], W["Wv"]], 0)) for W in layers]
    Wkvc = dev(np.stack([np.concatenate([W["Wkc"], W["Wvc"]], 0) for W in layers]))
    Wo = [dev(W["Wo"]) for W in layers]
    buf = dict(
        cu_q=torch.empty(P + 1, dtype=torch.int32, device=device),
        doc_of_pair=torch.empty(P, dtype=torch.int32, device=device),
        final_row=torch.empty(P, dtype=torch.int32, device=device),
        h0_final=torch.empty(P, dtype=torch.int32, device=device),
        h0_row=torch.empty(rows, dtype=torch.int32, device=device),
        pooled=torch.empty(D, Cmax, H, dtype=dt, device=device),
        chunk_mask=torch.empty(D, Cmax, dtype=torch.uint8, device=device),
        n_chunks=torch.empty(D, dtype=torch.int32, device=device),
        # cross K/V of every layer, row-major by passage chunk: [D, Cmax, L, 2*kv]
        kvc=torch.empty(D, Cmax, L, 2 * kv, dtype=dt, device=device),
        h=torch.empty(rows, H, dtype=torch.float32, device=device),
        qkv=torch.empty(rows, nqkv, dtype=dt, device=device),
        o=torch.empty(rows, sh.nq * sh.d, dtype=dt, device=device),
    )
    if dt == torch.bfloat16:
        buf["hb"] = torch.empty(rows, H, dtype=torch.bfloat16, device=device)
    U = int(lq.sum())  # decoder rows of the queries themselves
    buf.update(
        u_idx=torch.arange(U, dtype=torch.int32, device=device),
        p_idx=torch.arange(P, dtype=torch.int32, device=device),
        h0_copy=torch.empty(U, H, dtype=torch.float32, device=device),
        qkv_u=torch.empty(U, nqkv, dtype=dt, device=device),
        hf=torch.empty(P, H, dtype=torch.float32, device=device),
        qf=torch.empty(P, sh.nq * sh.d, dtype=dt, device=device),
        of=torch.empty(P, sh.nq * sh.d, dtype=dt, device=device),
        # row offsets of the queries' own rows and the queries' self partials
        cu_u=torch.empty(sh.n_queries + 1, dtype=torch.int32, device=device),
        o_self=torch.empty(U, sh.nq * sh.d, dtype=torch.float32, device=device),
        lse_self=torch.empty(U, sh.nq, dtype=torch.float32, device=device),
    )
    # split-KV workspace for the final rows of a one-layer stack (bf16)
    n_split = final_row_splits(P, sh.nq, sh.nkv, Cmax)
    if dt == torch.bfloat16 and L == 1 and n_split > 1:
        buf["split_ws"] = torch.empty(ops.split_workspace_bytes(n_split, P, sh.nq, sh.d), dtype=torch.uint8,
                                      device=device)
    if dt == torch.bfloat16:
        buf["h0b"] = torch.empty(U, H, dtype=torch.bfloat16, device=device)
        buf["hfb"] = torch.empty(P, H, dtype=torch.bfloat16, device=device)
    model = None
    if inputs.get("model"):
        mi = inputs["model"]
        I = int(mi["mlp_dim"])
        ch = min(rows, MLP_ROWS)
        model = dict(eps=float(mi["eps"]), theta=float(mi["rope_theta"]), I=I,
                     attn_norm=[dev(W["attn_norm"]) for W in layers], mlp_norm=[dev(W["mlp_norm"]) for W in layers],
                     Wgu=[dev(np.concatenate([W["Wg"], W["Wu"]], 0)) for W in layers],
                     Wd=[dev(W["Wd"]) for W in layers],
                     final_norm=dev(mi["final_norm"]) if mi.get("final_norm") is not None else None)
        buf.update(
            xn=torch.empty(rows, H, dtype=dt, device=device),       # normalised layer input, every row
            xu=torch.empty(U, H, dtype=dt, device=device),          # ... the queries' own rows
            xf=torch.empty(P, H, dtype=dt, device=device),          # ... the final rows
            hfn=torch.empty(P, H, dtype=torch.float32, device=device),  # final norm of the final rows
            m_x=torch.empty(ch, H, dtype=dt, device=device),        # MLP row chunk: normalised input,
            # gate | up projections (not needed when the fused kernel takes the width)
            m_gu=torch.empty(0 if dt == torch.bfloat16 and I % 128 == 0 else ch, 2 * I, dtype=dt, device=device),
            m_a=torch.empty(ch, I, dtype=dt, device=device),        # activation
        )
    return DeviceBatch(
        shape=sh, n_layers=L, dtype=dt, D=D, T=T, H=H, nq=sh.nq, nkv=sh.nkv, d=sh.d, chunk=chunk, Cmax=Cmax,
        n_queries=sh.n_queries, P=P, rows=rows, max_lq=int(lq.max()) if lq.size else 0,
        x=dev(inputs["x"]), token_mask=dev(inputs["token_mask"], torch.uint8), lq=dev(lq, torch.int32),
        h0=dev(inputs["h0"], torch.float32), Wqkv=Wqkv, Wkvc=Wkvc, Wo=Wo, w_yesno=dev(inputs["w_yesno"]), buf=buf,
        model=model)


MLP_ROWS = 1 << 16  # rows per gated-MLP pass (bounds the gate/up buffer)


def final_row_splits(P: int, nq: int, nkv: int, Cmax: int, cus: int = 256) -> int:
    """Shares of the cross keys for the final-row attention: enough workgroups
    for two per compute unit, at most one share per 32-chunk tile.  One
    workgroup takes a pair's final row for up to four query heads of one KV
    head."""
    groups = P * nkv * max(1, (nq // nkv) // 4)
    tiles = -(-Cmax // 32)
    return max(1, min(tiles, -(-2 * cus // max(1, groups)), 64))


def _no_rec(_name):
    return contextlib.nullcontext()


def front(b: DeviceBatch, stream=None, rec=_no_rec, h0_rows: bool = True):
    """Rows a0-a2: pair layout, chunk pooling and the cross K/V of every layer.
    ``rec(name)`` is an optional context-manager factory wrapped around each call
    (the benchmark records HIP events with it).  ``h0_rows`` = False skips the
    per-row residual-start index, which only a stack that computes every row
    of some layer reads."""
    B = b.buf
    lay = dict(cu_q=B["cu_q"], doc_of_pair=B["doc_of_pair"], final_row=B["final_row"], h0_row=B["h0_row"],
               h0_final=B["h0_final"], cu_u=B["cu_u"])
    _check = ops._check
    lib = ops.load()
    s = ops._stream(stream)
    with rec("pair_layout"):
        _check("kalm_pair_layout", lib.kalm_pair_layout(
            ops._ptr(b.lq), b.n_queries, b.D, ops._ptr(lay["cu_q"]), ops._ptr(lay["doc_of_pair"]),
            ops._ptr(lay["final_row"]), ops._ptr(lay["h0_row"]) if h0_rows else None, b.rows,
            ops._ptr(lay["h0_final"]), ops._ptr(lay["cu_u"]), s))
    with rec("chunk_pool"):
        ops.kalm_chunk_pool(b.x, b.token_mask, b.chunk, out=(B["pooled"], B["chunk_mask"], B["n_chunks"]),
                            stream=stream)
    with rec("cross_kv"):
        ops.kalm_cross_kv_layers(B["pooled"], B["chunk_mask"], b.Wkvc, out=B["kvc"], stream=stream)


def cross_layer(b: DeviceBatch, l: int) -> torch.Tensor:
    """Layer l's cross K/V [D*Cmax, 2*kv] (keys then values), a row-strided view of
    the all-layer buffer."""
    kv2 = 2 * b.nkv * b.d
    return b.buf["kvc"].view(b.D * b.Cmax, b.n_layers * kv2)[:, l * kv2:(l + 1) * kv2]


def pruned(b: DeviceBatch, prune: bool = True) -> bool:
    """Whether the last layer runs on final rows only (the score reads nothing else)."""
    return prune and b.n_layers >= 1


def decoder(b: DeviceBatch, stream=None, rec=_no_rec, prune: bool = True, reuse_self: bool = True,
            split_kv: bool = False):
    """Row a5 around a3: residual start, then every merged-attention layer.
    With ``prune`` and ``reuse_self`` the first layer computes each query's
    self-attention once and finishes every pair from it with the pair's cross
    keys (the merged softmax split at the self/cross boundary); ``split_kv``
    spreads those cross keys over several workgroups per pair in a one-layer
    stack with few pairs (off by default: at the one-query Nano shape the
    resumed pass is bound by per-workgroup start-up latency, not by its few
    key tiles, and the extra merge launch costs more than the split saves)."""
    if b.model is not None:
        return decoder_model(b, stream, rec, prune, reuse_self, split_kv)
    B = b.buf
    bf = b.dtype == torch.bfloat16
    qd, kv = b.nq * b.d, b.nkv * b.d
    # one pruned layer is both the first and the last: only the queries' own
    # rows and the pairs' final rows are ever computed
    single = prune and b.n_layers == 1
    if not prune:
        # residual start: every pair row from its query's first hidden state (the
        # pruned first layer instead adds its projection to those rows directly)
        with rec("gather_rows"):
            ops.kalm_gather_rows(b.h0, B["h0_row"], dst=B["h"], dst_bf16=B["hb"] if bf else None, stream=stream)
    qkv = B["qkv"]
    Q, Ks, Vs = qkv[:, :qd], qkv[:, qd:qd + kv], qkv[:, qd + kv:]
    scale = 1.0 / math.sqrt(b.d)
    last_pruned = pruned(b, prune)
    for l in range(b.n_layers):
        kvc = cross_layer(b, l)
        x_in = B["hb"] if bf else B["h"]
        if prune and l == 0:
            # the queries' own rows: one Q/K/V projection per query row, shared by its passages
            if bf:
                with rec("gather_query_rows"):
                    ops.kalm_gather_rows(b.h0, B["u_idx"], dst=B["h0_copy"], dst_bf16=B["h0b"], stream=stream)
            u = B["qkv_u"]
            with rec("qkv_linear_first"):
                ops.kalm_linear(B["h0b"] if bf else b.h0, b.Wqkv[0], Y=u, stream=stream)
            # every row of every pair, or (single layer) the final row of every pair
            rmode, o_rows, o_buf = ((ops.ROWS_SHARED_FINAL, b.P, B["of"]) if single
                                    else (ops.ROWS_SHARED, b.rows, B["o"]))
            if reuse_self:
                # the query's causal self-attention once, then each pair from it with its passage's cross keys
                with rec("self_attn_first"):
                    ops.kalm_self_attn_partial(u[:, :qd], u[:, qd:qd + kv], u[:, qd + kv:], B["cu_u"], b.max_lq,
                                               b.nq, b.nkv, b.d, scale=scale, out=B["o_self"], lse=B["lse_self"],
                                               stream=stream)
                if single and split_kv and "split_ws" in B:
                    # few pairs: each pair's cross keys in shares over more workgroups (split-KV)
                    with rec("merged_attn_first_split"):
                        ops.kalm_merged_attn_split(u[:, :qd], B["o_self"], B["lse_self"], B["cu_q"], b.max_lq,
                                                   kvc[:, :kv], kvc[:, kv:], B["chunk_mask"], B["doc_of_pair"],
                                                   b.nq, b.nkv, b.d, rmode, o_rows,
                                                   final_row_splits(b.P, b.nq, b.nkv, b.Cmax),
                                                   workspace=B["split_ws"], scale=scale, out=o_buf, stream=stream)
                else:
                    with rec("merged_attn_first_resume"):
                        ops.kalm_merged_attn_resume(u[:, :qd], B["o_self"], B["lse_self"], B["cu_q"], b.max_lq,
                                                    kvc[:, :kv], kvc[:, kv:], B["chunk_mask"], B["doc_of_pair"],
                                                    b.nq, b.nkv, b.d, rmode, o_rows, scale=scale, out=o_buf,
                                                    stream=stream)
            else:
                with rec("merged_attn_first"):
                    ops.kalm_merged_attn_rows(u[:, :qd], u[:, qd:qd + kv], u[:, qd + kv:], B["cu_q"], b.max_lq,
                                              kvc[:, :kv], kvc[:, kv:], B["chunk_mask"], B["doc_of_pair"], b.nq,
                                              b.nkv, b.d, rmode, o_rows, scale=scale, out=o_buf, stream=stream)
            if single:
                # each pair's residual starts from its query's final hidden state
                with rec("gather_final_rows"):
                    ops.kalm_gather_rows(b.h0, B["h0_final"], dst=B["hf"], stream=stream)
                with rec("o_linear_last"):
                    ops.kalm_linear(B["of"], b.Wo[l], Y=B["hf"], accumulate=True, stream=stream)
                continue
        elif last_pruned and l == b.n_layers - 1 and l > 0:
            # final rows only: self K/V of every row, Q / attention / projection of the final rows
            kvs = qkv.view(-1)[: b.rows * 2 * kv].view(b.rows, 2 * kv)
            with rec("kv_linear_last"):
                ops.kalm_linear(x_in, b.Wqkv[l][qd:], Y=kvs, stream=stream)
            with rec("gather_final_rows"):
                ops.kalm_gather_rows(B["h"], B["final_row"], dst=B["hf"], dst_bf16=B["hfb"] if bf else None,
                                     stream=stream)
            with rec("q_linear_last"):
                ops.kalm_linear(B["hfb"] if bf else B["hf"], b.Wqkv[l][:qd], Y=B["qf"], stream=stream)
            with rec("merged_attn_last"):
                ops.kalm_merged_attn_rows(B["qf"], kvs[:, :kv], kvs[:, kv:], B["cu_q"], b.max_lq, kvc[:, :kv],
                                          kvc[:, kv:], B["chunk_mask"], B["doc_of_pair"], b.nq, b.nkv, b.d,
                                          ops.ROWS_FINAL, b.P, scale=scale, out=B["of"], stream=stream)
            with rec("o_linear_last"):
                ops.kalm_linear(B["of"], b.Wo[l], Y=B["hf"], accumulate=True, stream=stream)
            continue
        else:
            with rec("qkv_linear"):
                ops.kalm_linear(x_in, b.Wqkv[l], Y=qkv, stream=stream)
            with rec("merged_attn"):
                ops.kalm_merged_attn(Q, Ks, Vs, B["cu_q"], b.max_lq, kvc[:, :kv], kvc[:, kv:], B["chunk_mask"],
                                     B["doc_of_pair"], b.nq, b.nkv, b.d, scale=scale, out=B["o"], stream=stream)
        if prune and l == 0:
            # residual start fused: h = h0[query row of each pair row] + O Wo^T
            with rec("o_linear_first"):
                ops.kalm_linear_residual(B["o"], b.Wo[l], b.h0, B["h0_row"], Y=B["h"],
                                         Y_bf16=B["hb"] if bf else None, stream=stream)
            continue
        with rec("o_linear"):
            ops.kalm_linear(B["o"], b.Wo[l], Y=B["h"], accumulate=True, Y_bf16=B["hb"] if bf else None,
                            stream=stream)


def decoder_model(b: DeviceBatch, stream=None, rec=_no_rec, prune: bool = True, reuse_self: bool = True,
                  split_kv: bool = False):
    """The model-shaped decoder layer around the merged attention: RMSNorm
    before the attention and before a gated-GELU MLP, RoPE on the self Q/K
    (positions 0..Lq-1 of each pair; the cached passage's cross keys carry
    none), residual adds in fp32.  The same row pruning as the plain stack
    (shared first layer with its self part once per query, final-row last
    layer, one-layer stacks on final rows only); the pairs' final rows end in
    ``hf``, the score reads their final RMSNorm."""
    B, M = b.buf, b.model
    qd, kv, eps, theta = b.nq * b.d, b.nkv * b.d, M["eps"], M["theta"]
    scale = 1.0 / math.sqrt(b.d)
    single = prune and b.n_layers == 1
    last_pruned = pruned(b, prune)
    I = M["I"]
    # the fused gate/up + activation kernel takes bf16 widths in blocks of 128 units
    fused_mlp = M["Wgu"][0].dtype == torch.bfloat16 and I % 128 == 0

    def norm(src, w, dst, name):
        with rec(name):
            ops.kalm_rms_norm(src, w, eps, out=dst, stream=stream)

    def rope(X, col0, nh, cu, mode, name):
        with rec(name):
            ops.kalm_rope(X, col0, nh, b.d, cu, b.max_lq, mode, theta, stream=stream)

    def mlp(h, l, tag=""):
        # gated MLP on the fp32 rows h (in place), MLP_ROWS rows per pass
        for r0 in range(0, h.shape[0], MLP_ROWS):
            hv = h[r0:r0 + MLP_ROWS]
            n = hv.shape[0]
            x, gu, a = B["m_x"][:n], B["m_gu"][:n], B["m_a"][:n]
            norm(hv, M["mlp_norm"][l], x, "mlp_norm" + tag)
            if fused_mlp:
                # gate/up projection and activation in one kernel: the [n, 2I]
                # projections never reach HBM
                with rec("mlp_gate_up_act" + tag):
                    ops.kalm_linear_gated_gelu(x, M["Wgu"][l][:I], M["Wgu"][l][I:], out=a, stream=stream)
            else:
                with rec("mlp_gate_up" + tag):
                    ops.kalm_linear(x, M["Wgu"][l], Y=gu, stream=stream)
                with rec("mlp_act" + tag):
                    ops.kalm_gated_gelu(gu, out=a, stream=stream)
            with rec("mlp_down" + tag):
                ops.kalm_linear(a, M["Wd"][l], Y=hv, accumulate=True, stream=stream)

    if not prune:
        with rec("gather_rows"):
            ops.kalm_gather_rows(b.h0, B["h0_row"], dst=B["h"], stream=stream)
    qkv = B["qkv"]
    for l in range(b.n_layers):
        kvc = cross_layer(b, l)
        cross = (kvc[:, :kv], kvc[:, kv:], B["chunk_mask"], B["doc_of_pair"], b.nq, b.nkv, b.d)
        if prune and l == 0:
            # the queries' own rows: norm, Q/K/V, RoPE once per query row
            u = B["qkv_u"]
            norm(b.h0, M["attn_norm"][0], B["xu"], "attn_norm_first")
            with rec("qkv_linear_first"):
                ops.kalm_linear(B["xu"], b.Wqkv[0], Y=u, stream=stream)
            rope(u, 0, b.nq, B["cu_u"], 0, "rope_q_first")
            rope(u, qd, b.nkv, B["cu_u"], 0, "rope_k_first")
            rmode, o_rows, o_buf = ((ops.ROWS_SHARED_FINAL, b.P, B["of"]) if single
                                    else (ops.ROWS_SHARED, b.rows, B["o"]))
            if reuse_self:
                with rec("self_attn_first"):
                    ops.kalm_self_attn_partial(u[:, :qd], u[:, qd:qd + kv], u[:, qd + kv:], B["cu_u"], b.max_lq,
                                               b.nq, b.nkv, b.d, scale=scale, out=B["o_self"], lse=B["lse_self"],
                                               stream=stream)
                if single and split_kv and "split_ws" in B:
                    with rec("merged_attn_first_split"):
                        ops.kalm_merged_attn_split(u[:, :qd], B["o_self"], B["lse_self"], B["cu_q"], b.max_lq,
                                                   *cross, rmode, o_rows, final_row_splits(b.P, b.nq, b.nkv, b.Cmax),
                                                   workspace=B["split_ws"], scale=scale, out=o_buf, stream=stream)
                else:
                    with rec("merged_attn_first_resume"):
                        ops.kalm_merged_attn_resume(u[:, :qd], B["o_self"], B["lse_self"], B["cu_q"], b.max_lq,
                                                    *cross, rmode, o_rows, scale=scale, out=o_buf, stream=stream)
            else:
                with rec("merged_attn_first"):
                    ops.kalm_merged_attn_rows(u[:, :qd], u[:, qd:qd + kv], u[:, qd + kv:], B["cu_q"], b.max_lq,
                                              *cross, rmode, o_rows, scale=scale, out=o_buf, stream=stream)
            if single:
                with rec("gather_final_rows"):
                    ops.kalm_gather_rows(b.h0, B["h0_final"], dst=B["hf"], stream=stream)
                with rec("o_linear_last"):
                    ops.kalm_linear(B["of"], b.Wo[0], Y=B["hf"], accumulate=True, stream=stream)
                mlp(B["hf"], 0, "_last")
                continue
        elif last_pruned and l == b.n_layers - 1 and l > 0:
            # final rows only: normalised K/V (RoPE on K) of every row; norm, Q, RoPE at the
            # final position, attention, projection and MLP of the final rows
            norm(B["h"], M["attn_norm"][l], B["xn"], "attn_norm")
            kvs = qkv.view(-1)[: b.rows * 2 * kv].view(b.rows, 2 * kv)
            with rec("kv_linear_last"):
                ops.kalm_linear(B["xn"], b.Wqkv[l][qd:], Y=kvs, stream=stream)
            rope(kvs, 0, b.nkv, B["cu_q"], 0, "rope_k")
            with rec("gather_final_rows"):
                ops.kalm_gather_rows(B["h"], B["final_row"], dst=B["hf"], stream=stream)
            norm(B["hf"], M["attn_norm"][l], B["xf"], "attn_norm_last")
            with rec("q_linear_last"):
                ops.kalm_linear(B["xf"], b.Wqkv[l][:qd], Y=B["qf"], stream=stream)
            rope(B["qf"], 0, b.nq, B["cu_q"], 1, "rope_q_last")
            with rec("merged_attn_last"):
                ops.kalm_merged_attn_rows(B["qf"], kvs[:, :kv], kvs[:, kv:], B["cu_q"], b.max_lq, *cross,
                                          ops.ROWS_FINAL, b.P, scale=scale, out=B["of"], stream=stream)
            with rec("o_linear_last"):
                ops.kalm_linear(B["of"], b.Wo[l], Y=B["hf"], accumulate=True, stream=stream)
            mlp(B["hf"], l, "_last")
            continue
        else:
            norm(B["h"], M["attn_norm"][l], B["xn"], "attn_norm")
            with rec("qkv_linear"):
                ops.kalm_linear(B["xn"], b.Wqkv[l], Y=qkv, stream=stream)
            rope(qkv, 0, b.nq, B["cu_q"], 0, "rope_q")
            rope(qkv, qd, b.nkv, B["cu_q"], 0, "rope_k")
            with rec("merged_attn"):
                ops.kalm_merged_attn(qkv[:, :qd], qkv[:, qd:qd + kv], qkv[:, qd + kv:], B["cu_q"], b.max_lq,
                                     *cross[:4], b.nq, b.nkv, b.d, scale=scale, out=B["o"], stream=stream)
        if prune and l == 0:
            # residual start fused: h = h0[query row of each pair row] + O Wo^T
            with rec("o_linear_first"):
                ops.kalm_linear_residual(B["o"], b.Wo[l], b.h0, B["h0_row"], Y=B["h"], stream=stream)
        else:
            with rec("o_linear"):
                ops.kalm_linear(B["o"], b.Wo[l], Y=B["h"], accumulate=True, stream=stream)
        mlp(B["h"], l)
    if not last_pruned:
        with rec("gather_final_rows"):
            ops.kalm_gather_rows(B["h"], B["final_row"], dst=B["hf"], stream=stream)


def score(b: DeviceBatch, stream=None, rec=_no_rec, prune: bool = True):
    """Row a4: yes/no readout at every pair's final row."""
    if b.model is not None:
        # the pairs' final rows are in hf; the readout follows the final RMSNorm when there is one
        hf = b.buf["hf"]
        if b.model["final_norm"] is not None:
            with rec("final_norm"):
                ops.kalm_rms_norm(hf, b.model["final_norm"], b.model["eps"], out=b.buf["hfn"], stream=stream)
            hf = b.buf["hfn"]
        with rec("yesno_score"):
            return ops.kalm_yesno_score(hf, b.buf["p_idx"], b.w_yesno, stream=stream)
    with rec("yesno_score"):
        if pruned(b, prune):
            return ops.kalm_yesno_score(b.buf["hf"], b.buf["p_idx"], b.w_yesno, stream=stream)
        return ops.kalm_yesno_score(b.buf["h"], b.buf["final_row"], b.w_yesno, stream=stream)


def step(b: DeviceBatch, stream=None, rec=_no_rec, prune: bool = True, reuse_self: bool = True,
         split_kv: bool = False):
    """One pass of the whole hot path over the batch; returns (yes, no, margin, score)."""
    front(b, stream, rec, h0_rows=not (prune and b.n_layers == 1))
    decoder(b, stream, rec, prune, reuse_self, split_kv)
    return score(b, stream, rec, prune)


def score_pairs(inputs: Dict[str, object], device="cuda", n_layers: Optional[int] = None, prune: bool = True,
                reuse_self: bool = True) -> Dict[str, torch.Tensor]:
    """Score every (query, passage) pair of one batch of host inputs, end to end on
    the device: the per-pair fields of the pages' scoring CLI -- the yes and no
    logits, their margin and score = sigmoid(margin) ("KaLM-Reranker-V1-Small
    Q4_K_M GGUF", Score a pair) -- each a device tensor [n_queries * n_docs] in
    pair order q * n_docs + d.  Larger margins rank first (``rerank.rerank``
    orders them on the device)."""
    b = upload(inputs, device, n_layers)
    yes, no, margin, sc = step(b, prune=prune, reuse_self=reuse_self)
    return {"yes_logit": yes, "no_logit": no, "margin": margin, "score": sc}


class StepGraph:
    """One step captured as a HIP graph (torch.cuda.CUDAGraph records the
    libkalm launches of ``step`` on its capture stream), so that a replay
    enqueues the whole hot path with one call: for the small workloads, whose
    kernels run for microseconds, the host-side launch cost otherwise sets the
    step time.  Every buffer the step writes is allocated by ``upload``
    beforehand and no libkalm call allocates, clears memory with a memset or
    synchronises, so the captured step is the eager step.  ``replay`` returns
    the (yes, no, margin, score) tensors the captured step wrote."""

    def __init__(self, b: DeviceBatch, prune: bool = True, reuse_self: bool = True, split_kv: bool = False):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):  # one eager step off the default stream before capture
            step(b, prune=prune, reuse_self=reuse_self, split_kv=split_kv)
        torch.cuda.current_stream().wait_stream(side)
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self.out = step(b, prune=prune, reuse_self=reuse_self, split_kv=split_kv)

    def replay(self):
        self.graph.replay()
        return self.out

