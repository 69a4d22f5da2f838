"""End-to-end GPU parity of the hot path (pool -> cross K/V -> merged-attention
stack -> yes/no score) against the oracle's mirror mode.

The GPU runs the whole batch exactly as bench.py times it (same entry points,
same launch configuration, full sizes); the oracle recomputes all pairs of the
small workloads and, for the stacks, one query against every passage (the
pages' validation compares a whole query's ranking) plus seeded random pairs
spread over queries and passages.  Per pair: the final hidden row element by
element (|g - r| <= 2e-2 + 1e-2 |r|; 1e-4 for the fp32 path), the score within
5e-3 (1e-4 fp32) and the margin; the a0 layout and the chunk counts/masks
bit-exact.  A noise-floor check compares the GPU and the mirror oracle with the
unrounded (pure fp64) oracle: the GPU's error must be of the size the bf16
storage itself causes (RMS within 1.5x, largest within 2x).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from encoder_decoder_document_amd import stack, synth
from parity_util import F32_TOL, SCORE_ATOL, assert_close, stack_tol, to_np

pytestmark = pytest.mark.gpu


def _sample_pairs(inp, k, seed=0, whole_query=None, doc_step=1):
    """Pairs to check: the longest/shortest query against the longest/shortest
    passage, the first and last pair, ``whole_query`` against every
    ``doc_step``-th passage, and seeded random pairs up to k more."""
    sh = inp["shape"]
    D = sh.n_docs
    lq = np.asarray(inp["lq"])
    dl = np.asarray(inp["doc_len"])
    qs = [int(np.argmax(lq)), int(np.argmin(lq))]
    ds = [int(np.argmax(dl)), int(np.argmin(dl))]
    picks = {qs[0] * D + ds[0], qs[1] * D + ds[1], qs[0] * D + ds[1], 0, sh.pairs - 1}
    if whole_query is not None:
        picks |= {whole_query * D + d for d in range(0, D, doc_step)}
    base = len(picks)
    rng = np.random.default_rng(seed)
    while len(picks) < min(base + k, sh.pairs):
        picks.add(int(rng.integers(0, sh.pairs)))
    return sorted(picks)


LAYOUT_KEYS = ("cu_q", "doc_of_pair", "final_row", "h0_final", "cu_u", "h0_row", "chunk_mask", "n_chunks")


def _run(inp):
    """The step on the GPU (bench.py's launch configuration); returns the batch
    and host copies of the per-pair outputs, each pair's final hidden row
    (the pruned step leaves them in hf, pair order) and the layout arrays."""
    b = stack.upload(inp)
    yes, no, margin, score = stack.step(b)
    torch.cuda.synchronize()
    got = dict(yes=to_np(yes), no=to_np(no), margin=to_np(margin), score=to_np(score), hf=to_np(b.buf["hf"]),
               n_layers=b.n_layers)
    got.update({k: b.buf[k].cpu().numpy() for k in LAYOUT_KEYS})
    return b, got


def _check(inp, got, pairs, hidden=True, n_layers=None):
    sh = inp["shape"]
    lay = oracle.pair_layout(inp["lq"], sh.n_docs)
    # a pruned one-layer step never reads the per-row index and leaves it unwritten
    keys = ("cu_q", "doc_of_pair", "final_row", "h0_final", "cu_u") + (("h0_row",) if got["n_layers"] > 1 else ())
    for k in keys:
        assert np.array_equal(got[k], lay[k]), k
    _, rcm, rnc = oracle.chunk_pool(np.zeros((sh.n_docs, sh.T, 1)), inp["token_mask"], sh.chunk)
    assert np.array_equal(got["chunk_mask"], rcm)
    assert np.array_equal(got["n_chunks"], rnc)
    ref = oracle.stack_scores(inp, pairs=pairs, mode="mirror", return_hidden=hidden, n_layers=n_layers)
    idx = np.asarray(pairs)
    if sh.dtype == "f32":
        for k in ("yes", "no", "margin", "score"):
            assert_close(got[k][idx], ref[k], *F32_TOL, k)
    else:
        assert_close(got["score"][idx], ref["score"], SCORE_ATOL, 0.0, "score")
        assert_close(got["margin"][idx], ref["margin"], 2e-2, 1e-2, "margin")
    if hidden:
        assert_close(got["hf"][idx], ref["h_final"], *stack_tol(sh.dtype), "final hidden rows")
    assert np.isfinite(got["score"]).all()
    return ref


@pytest.mark.parametrize("idx", [0, 1])
def test_stack_parity_all_pairs(idx):
    # the one-layer workloads: every pair
    sh = synth.SHAPES[idx]
    print(f"[case] stack {sh.name} all pairs", flush=True)
    inp = synth.make_inputs(idx, nan_padding=True)
    b, got = _run(inp)
    del b
    _check(inp, got, list(range(sh.pairs)))
    torch.cuda.empty_cache()


# The stacks at full size.  The GPU runs the whole batch once per workload
# and depth (cached on the host for the tests below); the oracle then checks
# one query against every passage (every second one for Long/wide, whose
# oracle takes about 1 s per pair and layer-third on the host) plus 16 seeded
# random pairs and the extreme pairs, in interleaved chunks so that no single
# test runs for minutes, and the noise floor against the unrounded oracle.
#
# Long/wide at its full 36 layers is checked by the noise floor only: its
# random stack without norms grows its residual updates layer after layer
# (update RMS 0.06 -> 0.7), which amplifies storage rounding about 40x, so the
# bf16-rounded oracle itself is up to 7e-3 from the exact score there (a
# margin difference of 0.08) -- two bf16 computations cannot agree to 5e-3 on
# every pair.  Its parity sample runs the full shape at 12 of the 36 layers,
# where the rounding noise stays well inside the tolerances.
SAMPLE = {2: (0, 1, 1), 3: (0, 1, 2), 4: (0, 2, 2)}   # workload: (whole query, passage step, chunks)
PARITY_LAYERS = {4: 12}
_INPUTS = {}
_RUNS = {}
_RANK = {}


def _full_size(idx, n_layers=None):
    if idx not in _INPUTS:
        _INPUTS.clear()  # one workload's inputs on the host at a time
        _RUNS.clear()
        _INPUTS[idx] = synth.make_inputs(idx, nan_padding=True)
    inp = _INPUTS[idx]
    if (idx, n_layers) not in _RUNS:
        b = stack.upload(inp, n_layers=n_layers)
        yes, no, margin, score = stack.step(b)
        torch.cuda.synchronize()
        got = dict(yes=to_np(yes), no=to_np(no), margin=to_np(margin), score=to_np(score), hf=to_np(b.buf["hf"]),
                   n_layers=b.n_layers)
        got.update({k: b.buf[k].cpu().numpy() for k in LAYOUT_KEYS})
        del b
        torch.cuda.empty_cache()
        wq, step, _ = SAMPLE[idx]
        _RUNS[(idx, n_layers)] = (got, _sample_pairs(inp, 16, whole_query=wq, doc_step=step))
    return (inp,) + _RUNS[(idx, n_layers)]


STACK_CASES = [(2, "parity", 0), (2, "noise", 0), (3, "parity", 0), (3, "parity", 1), (3, "noise", 0),
               (4, "parity", 0), (4, "parity", 1), (4, "noise", 0)]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("idx,kind,chunk", STACK_CASES)
def test_stack_full_size(idx, kind, chunk):
    sh = synth.SHAPES[idx]
    nl = PARITY_LAYERS.get(idx) if kind == "parity" else None
    print(f"[case] stack {sh.name} {kind} {chunk} layers={nl or sh.n_layers}", flush=True)
    inp, got, sample = _full_size(idx, nl)
    wq, step, n_chunks = SAMPLE[idx]
    D = sh.n_docs
    if kind == "parity":
        pairs = sample[chunk::n_chunks]
        print(f"[case] stack {sh.name}: oracle on {len(pairs)} of {len(sample)} sampled pairs", flush=True)
        ref = _check(inp, got, pairs, n_layers=nl)
        for p, r in zip(pairs, ref["score"]):
            if p // D == wq:
                _RANK.setdefault(idx, {})[p] = r
        if chunk == n_chunks - 1 and step == 1 and len(_RANK.get(idx, {})) == D:
            # the whole query's ranking: wherever the oracle's scores differ by
            # more than twice the score tolerance, the GPU orders the passages
            # the same way
            q = np.arange(wq * D, wq * D + D)
            r = np.asarray([_RANK[idx][p] for p in q])
            g = got["score"][q]
            resolvable = np.abs(r[:, None] - r[None, :]) > 2 * SCORE_ATOL
            inverted = np.sign(g[:, None] - g[None, :]) != np.sign(r[:, None] - r[None, :])
            assert not (resolvable & inverted).any(), "a resolvable pair of passages is ranked the other way"
        return
    # noise floor: the unrounded oracle (pure fp64, no bf16 storage) as the
    # common yardstick.  The GPU's score error against it must be of the size
    # the bf16 storage itself causes (the mirror oracle against pure): root
    # mean square within 1.5x, largest within 2x.  The GPU also rounds the
    # softmax weights of the PV product to bf16, which the mirror does not;
    # on the CPU that one rounding moves scores by about as much as all the
    # storage points together yet leaves the RMS against pure unchanged,
    # while the largest of a few dozen errors varies by 1.3-1.6x from it.
    pairs = _sample_pairs(inp, {2: 40, 3: 16, 4: 8}[idx], seed=11)
    mirror = oracle.stack_scores(inp, pairs=pairs, mode="mirror")
    pure = oracle.stack_scores(inp, pairs=pairs, mode="pure")
    d_gpu = np.abs(got["score"][np.asarray(pairs)] - pure["score"])
    d_mir = np.abs(mirror["score"] - pure["score"])
    rms = lambda d: float(np.sqrt(np.mean(d * d)))
    print(f"[case] noise floor {sh.name} ({len(pairs)} pairs): |gpu-pure| mean {d_gpu.mean():.3e} "
          f"rms {rms(d_gpu):.3e} max {d_gpu.max():.3e}; |mirror-pure| mean {d_mir.mean():.3e} "
          f"rms {rms(d_mir):.3e} max {d_mir.max():.3e}", flush=True)
    assert d_mir.max() > 0.0
    assert rms(d_gpu) <= 1.5 * rms(d_mir), (rms(d_gpu), rms(d_mir))
    assert d_gpu.max() <= 2.0 * d_mir.max(), (d_gpu.max(), d_mir.max())


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
    _check(inp, got, list(range(sh.pairs)))


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
    _check(inp, got, pairs)


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
    _check(inp, got, _sample_pairs(inp, 10))

