"""Seeded synthetic inputs for the reranker hot path.

This module only draws random numbers and lays them out; it holds none of
the method's arithmetic (no pooling, projection, attention or scoring), so
both the HIP path and the CPU oracle can be fed from it without sharing any
computation.

Shapes follow the five workload shapes of the KaLM-Reranker-V1 hot path:
passages of at most 1024 encoder tokens and queries of at most 512 decoder
tokens ("KaLM-Reranker-V1-Small Q4_K_M GGUF", Runtime boundaries), Nano
H=640 with 18 layers and Small H=1152 with 26 layers ("KaLM-Reranker-V1-Nano
-- MLX (Apple Silicon)", What this is), right-padded passages
("KaLM-Reranker-V1-Large Q8_0 GGUF", Frozen inference contract), and the
top-100-candidates-per-query shape of the FiQA run (Q4_K_M card, Complete
FIQA evaluation).  No dataset or trained weight is used: encoder states and
the first decoder hidden states are N(0,1), every weight is N(0, 0.02).

bf16 workloads: values are drawn in fp32 and rounded to the nearest bf16
(ties to even) here, so every array handed out holds values that bf16
represents exactly; they travel as float32 arrays and convert losslessly.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import numpy as np

__all__ = ["Shape", "SHAPES", "make_inputs", "round_to_bf16", "bf16_bits"]


@dataclasses.dataclass(frozen=True)
class Shape:
    name: str
    n_queries: int
    n_docs: int
    T: int                 # padded encoder length (tokens)
    H: int                 # hidden size
    nq: int                # query heads
    nkv: int               # key/value heads
    d: int                 # head dim
    n_layers: int
    dtype: str             # "f32" or "bf16"
    doc_len: tuple         # ("tiny_nonmult4", lo, hi) | ("loguniform", lo, hi) | ("const", n, n) | ("list", [..], 0)
    lq: tuple              # ("const", n, n) | ("uniform", lo, hi) | ("list", [..], 0)
    chunk: int = 4

    @property
    def pairs(self) -> int:
        return self.n_queries * self.n_docs


SHAPES: List[Shape] = [
    Shape("tiny_f32", 1, 8, 64, 64, 2, 1, 32, 1, "f32", ("tiny_nonmult4", 5, 64), ("const", 16, 16)),
    Shape("nano_1layer_bf16", 1, 100, 1024, 640, 4, 1, 256, 1, "bf16", ("loguniform", 32, 1024), ("const", 64, 64)),
    Shape("nano_stack18_bf16", 8, 100, 1024, 640, 4, 1, 256, 18, "bf16", ("loguniform", 32, 1024), ("uniform", 32, 128)),
    Shape("small_stack26_bf16", 32, 100, 1024, 1152, 4, 1, 256, 26, "bf16", ("loguniform", 64, 1024), ("uniform", 64, 512)),
    Shape("long_wide36_bf16", 64, 100, 1024, 2560, 8, 4, 256, 36, "bf16", ("const", 1024, 1024), ("const", 512, 512)),
]


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 value (ties to even), returned as float32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    r = (u >> 16) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u                      # wraps only for NaN bit patterns, restored below
    r &= np.uint32(0xFFFF0000)
    out = r.view(np.float32)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = np.nan
    return out


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that bf16 represents exactly (uint16 array)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return (a.view(np.uint32) >> 16).astype(np.uint16)


def _doc_lengths(rng: np.random.Generator, spec: tuple, D: int) -> np.ndarray:
    kind, lo, hi = spec
    if kind == "tiny_nonmult4":
        choices = np.array([v for v in range(lo, hi + 1) if v % 4 != 0], dtype=np.int64)
        return rng.choice(choices, size=D).astype(np.int32)
    if kind == "loguniform":
        u = rng.uniform(math.log(lo), math.log(hi + 1), size=D)
        return np.minimum(hi, np.floor(np.exp(u))).astype(np.int32)
    if kind == "const":
        return np.full(D, lo, dtype=np.int32)
    if kind == "list":
        return np.resize(np.asarray(lo, dtype=np.int32), D)
    raise ValueError(kind)


def _query_lengths(rng: np.random.Generator, spec: tuple, Q: int) -> np.ndarray:
    kind, lo, hi = spec
    if kind == "const":
        return np.full(Q, lo, dtype=np.int32)
    if kind == "uniform":
        return rng.integers(lo, hi + 1, size=Q).astype(np.int32)
    if kind == "list":
        return np.resize(np.asarray(lo, dtype=np.int32), Q)
    raise ValueError(kind)


def _normal(rng: np.random.Generator, shape, std: float, bf16: bool) -> np.ndarray:
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return round_to_bf16(a) if bf16 else a


def make_inputs(shape_index: int, seed: Optional[int] = None, nan_padding: bool = True,
                n_layers: Optional[int] = None, shape: Optional[Shape] = None,
                mlp_dim: Optional[int] = None) -> Dict[str, object]:
    """Draw one batch for ``SHAPES[shape_index]`` (or an explicit ``shape``).

    Returns a dict of host arrays:
      doc_len [D] int32, token_mask [D,T] uint8 (prefix masks, right padding),
      x [D,T,H] float32 (padding positions NaN when ``nan_padding`` else 0),
      lq [Q] int32, h0 [sum(lq), H] float32 (query q's rows are contiguous,
      in query order), per-layer weight dicts ``layers[l]`` with
      Wq [nq*d,H], Wk/Wv [nkv*d,H], Wkc/Wvc [nkv*d,H], Wo [H,nq*d], and
      w_yesno [2,H] (row 0 stands for the "yes" LM-head row, row 1 for "no").
    The seed defaults to 1000 + shape_index.  ``n_layers`` overrides the layer
    count (tests use it to cut long stacks).

    With ``mlp_dim`` = I the batch also carries the weights of a model-shaped
    layer, drawn from a generator of their own so that every array above is
    unchanged: per layer attn_norm and mlp_norm [H] (1 + N(0, 0.1^2)), Wg and
    Wu [I,H] and Wd [H,I] (N(0, 0.02^2)), and ``model`` = dict(rope_theta
    10000, eps 1e-6, final_norm [H] (1 + N(0, 0.1^2))).
    """
    sh = shape if shape is not None else SHAPES[shape_index]
    if seed is None:
        seed = 1000 + shape_index
    L = sh.n_layers if n_layers is None else n_layers
    bf16 = sh.dtype == "bf16"
    streams = np.random.SeedSequence(seed).spawn(6)
    g_len, g_lq, g_x, g_h0, g_w, g_yn = [np.random.Generator(np.random.PCG64(s)) for s in streams]

    D, T, H = sh.n_docs, sh.T, sh.H
    doc_len = _doc_lengths(g_len, sh.doc_len, D)
    token_mask = (np.arange(T)[None, :] < doc_len[:, None]).astype(np.uint8)
    x = _normal(g_x, (D, T, H), 1.0, bf16)
    x[token_mask == 0] = np.nan if nan_padding else 0.0

    lq = _query_lengths(g_lq, sh.lq, sh.n_queries)
    h0 = g_h0.standard_normal(size=(int(lq.sum()), H), dtype=np.float32)

    layers = []
    for _ in range(L):
        layers.append(dict(
            Wq=_normal(g_w, (sh.nq * sh.d, H), 0.02, bf16),
            Wk=_normal(g_w, (sh.nkv * sh.d, H), 0.02, bf16),
            Wv=_normal(g_w, (sh.nkv * sh.d, H), 0.02, bf16),
            Wkc=_normal(g_w, (sh.nkv * sh.d, H), 0.02, bf16),
            Wvc=_normal(g_w, (sh.nkv * sh.d, H), 0.02, bf16),
            Wo=_normal(g_w, (H, sh.nq * sh.d), 0.02, bf16),
        ))
    w_yesno = _normal(g_yn, (2, H), 0.02, bf16)
    out = dict(shape=sh, seed=seed, doc_len=doc_len, token_mask=token_mask, x=x,
               lq=lq, h0=h0, layers=layers, w_yesno=w_yesno)
    if mlp_dim:
        g_m = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 7])))
        I = int(mlp_dim)
        for W in layers:
            W.update(attn_norm=1.0 + _normal(g_m, (H,), 0.1, bf16), mlp_norm=1.0 + _normal(g_m, (H,), 0.1, bf16),
                     Wg=_normal(g_m, (I, H), 0.02, bf16), Wu=_normal(g_m, (I, H), 0.02, bf16),
                     Wd=_normal(g_m, (H, I), 0.02, bf16))
            if bf16:  # 1 + x must stay bf16-representable
                W["attn_norm"] = round_to_bf16(W["attn_norm"])
                W["mlp_norm"] = round_to_bf16(W["mlp_norm"])
        fn = 1.0 + _normal(g_m, (H,), 0.1, bf16)
        out["model"] = dict(rope_theta=10000.0, eps=1e-6, final_norm=round_to_bf16(fn) if bf16 else fn,
                            mlp_dim=I)
    return out


def normal(seed: int, shape, std: float = 1.0, bf16: bool = True) -> np.ndarray:
    """Seeded N(0, std^2) array (float32; bf16-representable when ``bf16``)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return _normal(rng, shape, std, bf16)


def integers(seed: int, lo: int, hi: int, size) -> np.ndarray:
    """Seeded uniform integers in [lo, hi] (int32)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.integers(lo, hi + 1, size=size).astype(np.int32)


def bernoulli_mask(seed: int, p: float, shape) -> np.ndarray:
    """Seeded 0/1 uint8 mask with P(1) = p."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return (rng.random(shape) < p).astype(np.uint8)
