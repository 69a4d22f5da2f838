"""End-to-end GPU parity of the hot path (pool -> cross K/V -> merged-attention
stack -> yes/no score) against the oracle's mirror mode.

The GPU runs the whole batch exactly as bench.py times it (same entry points,
same launch configuration, full sizes); the oracle recomputes all pairs of the
small workloads and a sample of pairs (longest/shortest query, longest/
shortest passage, first/last, seeded random) of the large ones.  Scores must
agree within 5e-3 (bf16 storage) or 1e-4 (fp32 path); the a0 layout and the
chunk counts/masks must be bit-exact.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from encoder_decoder_document_amd import stack, synth
from parity_util import F32_TOL, SCORE_ATOL, assert_close, to_np

pytestmark = pytest.mark.gpu


def _sample_pairs(inp, k, seed=0):
    sh = inp["shape"]
    D = sh.n_docs
    lq = np.asarray(inp["lq"])
    dl = np.asarray(inp["doc_len"])
    qs = [int(np.argmax(lq)), int(np.argmin(lq))]
    ds = [int(np.argmax(dl)), int(np.argmin(dl))]
    picks = {qs[0] * D + ds[0], qs[1] * D + ds[1], qs[0] * D + ds[1], 0, sh.pairs - 1}
    rng = np.random.default_rng(seed)
    while len(picks) < k:
        picks.add(int(rng.integers(0, sh.pairs)))
    return sorted(picks)[:max(k, 1)] if k < len(picks) else sorted(picks)


def _run(inp):
    b = stack.upload(inp)
    yes, no, margin, score = stack.step(b)
    torch.cuda.synchronize()
    return b, dict(yes=to_np(yes), no=to_np(no), margin=to_np(margin), score=to_np(score))


def _check(inp, b, got, pairs):
    sh = inp["shape"]
    lay = oracle.pair_layout(inp["lq"], sh.n_docs)
    # a pruned one-layer step never reads the per-row index and leaves it unwritten
    keys = ("cu_q", "doc_of_pair", "final_row", "h0_final", "cu_u") + (("h0_row",) if b.n_layers > 1 else ())
    for k in keys:
        assert np.array_equal(b.buf[k].cpu().numpy(), lay[k]), k
    _, rcm, rnc = oracle.chunk_pool(np.zeros((sh.n_docs, sh.T, 1)), inp["token_mask"], sh.chunk)
    assert np.array_equal(b.buf["chunk_mask"].cpu().numpy(), rcm)
    assert np.array_equal(b.buf["n_chunks"].cpu().numpy(), rnc)
    ref = oracle.stack_scores(inp, pairs=pairs, mode="mirror")
    idx = np.asarray(pairs)
    if sh.dtype == "f32":
        for k in ("yes", "no", "margin", "score"):
            assert_close(got[k][idx], ref[k], *F32_TOL, k)
    else:
        assert_close(got["score"][idx], ref["score"], SCORE_ATOL, 0.0, "score")
        assert_close(got["margin"][idx], ref["margin"], 2e-2, 1e-2, "margin")
    assert np.isfinite(got["score"]).all()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("idx,n_sample", [(0, None), (1, None), (2, 16), (3, 6), (4, 2)])
def test_stack_parity(idx, n_sample):
    sh = synth.SHAPES[idx]
    print(f"[case] stack {sh.name} sample={n_sample}", flush=True)
    inp = synth.make_inputs(idx, nan_padding=True)
    b, got = _run(inp)
    pairs = list(range(sh.pairs)) if n_sample is None else _sample_pairs(inp, n_sample)
    _check(inp, b, got, pairs)
    del b
    torch.cuda.empty_cache()


def test_score_pairs_fields_and_ranking():
    # the one-call API: the per-pair fields of the scoring CLI, equal to the
    # step's outputs, and the ranking above it ordered by margin (= by score)
    sh = synth.SHAPES[1]
    print(f"[case] score_pairs {sh.name}", flush=True)
    inp = synth.make_inputs(1, nan_padding=True)
    out = stack.score_pairs(inp)
    assert set(out) == {"yes_logit", "no_logit", "margin", "score"}
    got = {k: to_np(v) for k, v in out.items()}
    ref = oracle.stack_scores(inp, pairs=list(range(sh.pairs)), mode="mirror")
    assert_close(got["score"], ref["score"], SCORE_ATOL, 0.0, "score")
    assert_close(got["margin"], ref["margin"], 2e-2, 1e-2, "margin")
    assert np.allclose(got["margin"], got["yes_logit"] - got["no_logit"], rtol=0, atol=1e-5)
    from encoder_decoder_document_amd import rerank
    recs = rerank.rerank(out["score"], sh.n_docs, 5)
    assert len(recs) == sh.n_queries and all(len(r) == 5 for r in recs)
    for q, r in enumerate(recs):
        s = got["score"][q * sh.n_docs:(q + 1) * sh.n_docs]
        assert [x["index"] for x in r] == list(np.argsort(-s, kind="stable")[:5])


def test_stack_edge_empty_and_one_token_passages():
    # a passage with no valid token leaves pure causal self-attention; a 1-token
    # passage pools to that token; queries of length 1 read their only row
    sh = synth.Shape("edge_bf16", 3, 5, 40, 256, 4, 1, 256, 2, "bf16", ("list", [0, 1, 5, 40, 17], 0),
                     ("list", [1, 33, 7], 0))
    print(f"[case] stack {sh.name}", flush=True)
    inp = synth.make_inputs(0, seed=77, shape=sh)
    b, got = _run(inp)
    _check(inp, b, got, list(range(sh.pairs)))


@pytest.mark.parametrize("reuse_self", [True, False])
def test_stack_pruned_path_equals_full_path(reuse_self):
    # the shared first layer (with or without its self part computed once per
    # query) and the final-row last layer change how much is computed, not the
    # result: scores of both paths agree, and with the oracle
    idx = 2
    sh = synth.SHAPES[idx]
    print(f"[case] stack {sh.name} 3 layers, pruned (reuse_self={reuse_self}) vs full", flush=True)
    inp = synth.make_inputs(idx, nan_padding=True, n_layers=3)
    b = stack.upload(inp)
    full = to_np(stack.step(b, prune=False)[3])
    pruned = to_np(stack.step(b, prune=True, reuse_self=reuse_self)[3])
    torch.cuda.synchronize()
    assert_close(pruned, full, 1e-3, 0.0, "pruned vs full score")
    pairs = _sample_pairs(inp, 8)
    ref = oracle.stack_scores(inp, pairs=pairs, mode="mirror")
    assert_close(pruned[np.asarray(pairs)], ref["score"], SCORE_ATOL, 0.0, "pruned score vs oracle")


@pytest.mark.parametrize("reuse_self,split_kv", [(True, False), (True, True), (False, False)])
def test_stack_single_layer_pruned_equals_full(reuse_self, split_kv):
    # one layer is both the first and the last: the pruned path computes the
    # queries' own rows and each pair's final row only; the scores agree with
    # the path that computes every row, and with the oracle
    idx = 1
    sh = synth.SHAPES[idx]
    print(f"[case] stack {sh.name} single layer, pruned (reuse_self={reuse_self}, split_kv={split_kv}) vs full",
          flush=True)
    inp = synth.make_inputs(idx, nan_padding=True)
    b = stack.upload(inp)
    assert "split_ws" in b.buf  # 100 pairs: the split-KV workspace exists
    full = to_np(stack.step(b, prune=False)[3])
    pruned = to_np(stack.step(b, prune=True, reuse_self=reuse_self, split_kv=split_kv)[3])
    torch.cuda.synchronize()
    assert_close(pruned, full, 1e-3, 0.0, "pruned vs full score")
    pairs = _sample_pairs(inp, 8)
    ref = oracle.stack_scores(inp, pairs=pairs, mode="mirror")
    assert_close(pruned[np.asarray(pairs)], ref["score"], SCORE_ATOL, 0.0, "pruned score vs oracle")


@pytest.mark.parametrize("idx,n_layers", [(1, None), (2, 3)])
def test_step_graph_replays_equal_eager(idx, n_layers):
    # the step captured as a HIP graph: every replay, with eager work and
    # synchronisations between replays, gives the eager step's scores exactly
    sh = synth.SHAPES[idx]
    print(f"[case] step graph {sh.name} layers={n_layers}", flush=True)
    inp = synth.make_inputs(idx, nan_padding=True, n_layers=n_layers)
    b = stack.upload(inp)
    eager = [to_np(t).copy() for t in stack.step(b)]
    torch.cuda.synchronize()
    g = stack.StepGraph(b)
    for i in range(3):
        out = [to_np(t) for t in g.replay()]
        torch.cuda.synchronize()
        for k, (x, y) in enumerate(zip(out, eager)):
            assert np.array_equal(x, y, equal_nan=True), f"replay {i} output {k}"
        again = to_np(stack.step(b)[3])  # eager work between replays
        torch.cuda.synchronize()
        assert np.array_equal(again, eager[3], equal_nan=True)


@pytest.mark.parametrize("idx,n_layers,mlp_dim,n_sample", [(0, 2, 96, None), (1, None, 1536, 8), (2, 3, 1536, 8)])
def test_model_shaped_stack_parity(idx, n_layers, mlp_dim, n_sample):
    # the model-shaped layer (RMSNorm, RoPE on the self Q/K, gated-GELU MLP,
    # final norm) through the pruned path, against the oracle
    sh = synth.SHAPES[idx]
    print(f"[case] model-shaped stack {sh.name} layers={n_layers} mlp={mlp_dim}", flush=True)
    inp = synth.make_inputs(idx, nan_padding=True, n_layers=n_layers, mlp_dim=mlp_dim)
    b, got = _run(inp)
    pairs = list(range(sh.pairs)) if n_sample is None else _sample_pairs(inp, n_sample)
    _check(inp, b, got, pairs)


def test_model_shaped_pruned_equals_full():
    idx = 2
    sh = synth.SHAPES[idx]
    print(f"[case] model-shaped stack {sh.name} 3 layers, pruned vs full", flush=True)
    inp = synth.make_inputs(idx, nan_padding=True, n_layers=3, mlp_dim=1536)
    b = stack.upload(inp)
    full = to_np(stack.step(b, prune=False)[3])
    pruned = to_np(stack.step(b, prune=True)[3])
    torch.cuda.synchronize()
    assert_close(pruned, full, 1e-3, 0.0, "pruned vs full score (model-shaped)")


@pytest.mark.parametrize("chunk", [1, 2, 8, 16])
def test_stack_matryoshka_chunk_sizes(chunk):
    # the pooling granularity is a parameter of the path: every chunk size
    # flows through pooling, cross K/V and the merged attention (Cmax = T / chunk)
    import dataclasses
    base = synth.SHAPES[2]
    sh = dataclasses.replace(base, name=f"nano_chunk{chunk}", n_queries=2, n_layers=2, chunk=chunk)
    print(f"[case] stack {sh.name}", flush=True)
    inp = synth.make_inputs(0, seed=300 + chunk, shape=sh)
    b, got = _run(inp)
    assert b.Cmax == -(-sh.T // chunk)
    _check(inp, b, got, _sample_pairs(inp, 10))

