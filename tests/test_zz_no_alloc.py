"""kalm_merged_attn_split_noalloc against kalm_merged_attn_split (GPU).

The no-allocation entry point keeps the split-KV partials in the library's
static device scratch instead of a caller workspace; on the same inputs it
must give exactly the workspace version's outputs (the same kernels run), on
two calls in a row -- the second one smaller, so stale partials of the first
call would show if any slot the merge reads were left unwritten.
"""
import numpy as np
import pytest
import torch

from encoder_decoder_document_amd import ops, synth
from parity_util import to_dev

pytestmark = pytest.mark.gpu


def _case(seed, lq, D, Cmax, nq, nkv, row_mode, d=256):
    lq = np.asarray(lq, np.int32)
    rng = np.random.default_rng(seed)
    docs_c = rng.integers(0, Cmax + 1, D)
    docs_c[0] = Cmax
    U = int(lq.sum())
    bf = torch.bfloat16
    Qu = to_dev(synth.normal(seed + 1, (U, nq * d), 0.7, True), bf)
    Ku = to_dev(synth.normal(seed + 2, (U, nkv * d), 0.7, True), bf)
    Vu = to_dev(synth.normal(seed + 3, (U, nkv * d), 1.0, True), bf)
    cm = (np.arange(Cmax)[None] < docs_c[:, None]).astype(np.uint8)
    Kc = synth.normal(seed + 4, (D * Cmax, nkv * d), 0.7, True)
    Vc = synth.normal(seed + 5, (D * Cmax, nkv * d), 1.0, True)
    lay = ops.kalm_pair_layout(to_dev(lq, torch.int32), D, rows=int(D * U))
    lay1 = ops.kalm_pair_layout(to_dev(lq, torch.int32), 1, with_h0_row=False)
    sO, sL = ops.kalm_self_attn_partial(Qu, Ku, Vu, lay1["cu_q"], int(lq.max()), nq, nkv, d)
    P = len(lq) * D
    o_rows = P if row_mode == ops.ROWS_SHARED_FINAL else int(D * U)
    return dict(args=(Qu, sO, sL, lay["cu_q"], int(lq.max()), to_dev(Kc, bf), to_dev(Vc, bf),
                      to_dev(cm, torch.uint8), lay["doc_of_pair"], nq, nkv, d, row_mode, o_rows),
                o_rows=o_rows, nq=nq, d=d)


def _compare(c, n_split):
    o_rows, nq, d = c["o_rows"], c["nq"], c["d"]
    lse_ref = torch.empty(o_rows, nq, dtype=torch.float32, device="cuda")
    ref = ops.kalm_merged_attn_split(*c["args"], n_split, lse=lse_ref)
    out = torch.full((o_rows, nq * d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((o_rows, nq), float("nan"), dtype=torch.float32, device="cuda")
    ops.kalm_merged_attn_split_noalloc(*c["args"], n_split, out=out, lse=lse)
    torch.cuda.synchronize()
    assert torch.isfinite(ref.float()).all()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), "O differs from the workspace version"
    assert torch.equal(lse, lse_ref), "lse differs from the workspace version"


def test_noalloc_split_equals_workspace_split_on_two_calls():
    print("[case] no-alloc split: one query x 100 passages (final rows), then a smaller GQA batch", flush=True)
    big = _case(81, [64], 100, 256, 4, 1, ops.ROWS_SHARED_FINAL)
    small = _case(91, [9, 30], 7, 96, 8, 4, ops.ROWS_SHARED)
    assert ops.split_workspace_bytes(8, big["o_rows"], 4, 256) <= ops.NOALLOC_SCRATCH_BYTES
    _compare(big, 8)
    _compare(small, 3)
    _compare(big, 2)   # back to the large batch with another share count
