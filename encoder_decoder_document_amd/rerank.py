"""Ranking above the hot path: each query's passages by relevance score.

``rerank(score, n_docs, top_n)`` turns the per-pair scores of a batch (pair
order q * n_docs + d, as ``stack.step`` returns them) into, per query, the
top_n passages highest score first as ``{"index", "relevance_score"}``
records -- the shape of the pages' ``rerank(query, docs, top_n)`` result
("KaLM-Reranker-V1-Nano -- MLX (Apple Silicon)", Files).  The ordering runs
on the GPU (kalm_rank_topn); this module only reshapes and converts.
"""
from __future__ import annotations

from typing import Dict, List

import torch

from . import ops


def rank_topn(score: torch.Tensor, n_docs: int, top_n: int):
    """score [n_queries * n_docs] (pair order) -> (index, score) [n_queries, top_n] on the device."""
    s = score.reshape(-1, n_docs).contiguous()
    return ops.kalm_rank_topn(s, top_n)


def rerank(score: torch.Tensor, n_docs: int, top_n: int) -> List[List[Dict[str, float]]]:
    """Per query, the top_n passages best first: [{"index": d, "relevance_score": s}, ...]."""
    idx, val = rank_topn(score, n_docs, top_n)
    return [[{"index": int(i), "relevance_score": float(v)} for i, v in zip(ri, rv)]
            for ri, rv in zip(idx.cpu().tolist(), val.cpu().tolist())]
