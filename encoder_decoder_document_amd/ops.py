"""Thin Python binding of libkalm (argument marshalling only).

Every function has the name of the C entry point it wraps, takes torch tensors
that already live on the GPU, passes their device pointers and the current
HIP stream, and raises ``KalmError`` on a non-OK status.  No computation of
the hot path happens here; PyTorch only supplies device memory and streams.
The library is loaded from the package directory (libkalm.so, or the debug
build libkalm_debug.so when the environment variable KALM_LIBRARY is "debug";
any other value is taken as a path); when it is missing (or no GPU is usable)
the calls fail loudly -- there is no CPU fallback.
"""
from __future__ import annotations

import contextlib
import ctypes
import math
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
RELEASE_LIB_PATH = os.path.join(_PKG, "libkalm.so")
DEBUG_LIB_PATH = os.path.join(_PKG, "libkalm_debug.so")
_env_lib = os.environ.get("KALM_LIBRARY", "")
_LIB_PATH = DEBUG_LIB_PATH if _env_lib == "debug" else (_env_lib or RELEASE_LIB_PATH)
_lib = None

KALM_OK, KALM_ERR_INVALID_ARG, KALM_ERR_UNSUPPORTED, KALM_ERR_NO_DEVICE, KALM_ERR_LAUNCH, KALM_ERR_BOUNDS = range(6)
KALM_F32, KALM_BF16 = 0, 1

_c_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_f32 = ctypes.c_float

_SIGS = {
    "kalm_version": (_i32, []),
    "kalm_last_error": (ctypes.c_char_p, []),
    "kalm_debug_build": (_i32, []),
    "kalm_device_check": (_i32, []),
    "kalm_pair_layout": (_i32, [_c_p, _i32, _i32, _c_p, _c_p, _c_p, _c_p, _i64, _c_p, _c_p, _c_p]),
    "kalm_chunk_pool": (_i32, [_c_p, _c_p, _i32, _i32, _i32, _i32, _i32, _c_p, _c_p, _c_p, _c_p]),
    "kalm_cross_kv": (_i32, [_c_p, _c_p, _i32, _i32, _i32, _c_p, _i32, _i32, _c_p, _c_p]),
    "kalm_cross_kv_layers": (_i32, [_c_p, _c_p, _i32, _i32, _i32, _c_p, _i32, _i32, _i32, _c_p, _c_p]),
    "kalm_merged_attn": (_i32, [_c_p, _i64, _c_p, _c_p, _i64, _c_p, _i32, _i64, _i32, _c_p, _c_p, _i64,
                                _c_p, _c_p, _i32, _i32, _i32, _i32, _i32, _f32, _i32, _c_p, _i64, _c_p, _c_p]),
    "kalm_merged_attn_rows": (_i32, [_c_p, _i64, _i64, _c_p, _c_p, _i64, _i64, _c_p, _i32, _i32, _c_p, _c_p, _i64,
                                     _c_p, _c_p, _i32, _i32, _i32, _i32, _i32, _f32, _i32, _c_p, _i64, _i64, _c_p,
                                     _i32, _c_p]),
    "kalm_self_attn_partial": (_i32, [_c_p, _i64, _c_p, _c_p, _i64, _i64, _c_p, _i32, _i32, _i32, _i32, _i32, _f32,
                                      _i32, _c_p, _i64, _c_p, _c_p]),
    "kalm_merged_attn_resume": (_i32, [_c_p, _i64, _i64, _c_p, _i64, _c_p, _c_p, _i32, _i32, _c_p, _c_p, _i64, _c_p,
                                       _c_p, _i32, _i32, _i32, _i32, _i32, _f32, _i32, _c_p, _i64, _i64, _c_p, _i32,
                                       _c_p]),
    "kalm_merged_attn_split": (_i32, [_c_p, _i64, _i64, _c_p, _i64, _c_p, _c_p, _i32, _i32, _c_p, _c_p, _i64, _c_p,
                                      _c_p, _i32, _i32, _i32, _i32, _i32, _f32, _i32, _c_p, _i64, _i64, _c_p, _i32,
                                      _i32, _c_p, _i64, _c_p]),
    "kalm_merged_attn_split_noalloc": (_i32, [_c_p, _i64, _i64, _c_p, _i64, _c_p, _c_p, _i32, _i32, _c_p, _c_p, _i64,
                                              _c_p, _c_p, _i32, _i32, _i32, _i32, _i32, _f32, _i32, _c_p, _i64, _i64,
                                              _c_p, _i32, _i32, _c_p]),
    "kalm_rms_norm": (_i32, [_c_p, _i32, _i64, _i64, _i32, _c_p, _i32, _f32, _c_p, _i32, _i64, _c_p]),
    "kalm_rope": (_i32, [_c_p, _i32, _i64, _i64, _i32, _i32, _i32, _c_p, _i32, _i32, _i32, _f32, _c_p]),
    "kalm_gated_gelu": (_i32, [_c_p, _i32, _i64, _i64, _i32, _c_p, _i64, _c_p]),
    "kalm_linear_gated_gelu": (_i32, [_c_p, _c_p, _c_p, _i32, _i32, _i32, _c_p, _c_p]),
    "kalm_yesno_score": (_i32, [_c_p, _i32, _i64, _i64, _c_p, _i32, _i32, _c_p, _i32, _c_p, _c_p, _c_p, _c_p, _c_p]),
    "kalm_linear": (_i32, [_c_p, _c_p, _i32, _i32, _i32, _i32, _c_p, _i32, _i32, _c_p, _c_p]),
    "kalm_linear_residual": (_i32, [_c_p, _c_p, _i32, _i32, _i32, _i32, _c_p, _c_p, _i64, _c_p, _c_p, _c_p]),
    "kalm_gather_rows": (_i32, [_c_p, _c_p, _i64, _i32, _i64, _c_p, _c_p, _c_p]),
    "kalm_rank_topn": (_i32, [_c_p, _i32, _i32, _i32, _c_p, _c_p, _c_p]),
}

EXPORTED = tuple(_SIGS)


class KalmError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


def lib_path() -> str:
    return _LIB_PATH


def load(path: Optional[str] = None):
    """Load libkalm.so (once) and declare every entry point's signature."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or _LIB_PATH
    if not os.path.exists(p):
        raise FileNotFoundError(f"{os.path.basename(p)} not built at {p}; run __graft_entry__.build() first")
    lib = ctypes.CDLL(p)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


@contextlib.contextmanager
def using(path: str):
    """Route every call made inside the block through the library at `path`
    (for example DEBUG_LIB_PATH), then restore the previous one."""
    global _lib, _LIB_PATH
    prev, prev_path = load(), _LIB_PATH
    _lib, _LIB_PATH = load(path), path
    try:
        yield _lib
    finally:
        _lib, _LIB_PATH = prev, prev_path


def debug_build() -> bool:
    return bool(load().kalm_debug_build())


def _check(fn: str, status: int):
    if status != KALM_OK:
        raise KalmError(fn, status, load().kalm_last_error().decode())


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return KALM_F32
    if t.dtype == torch.bfloat16:
        return KALM_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libkalm takes device tensors only")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream or None


def _contig(*ts):
    for t in ts:
        if t is not None and not t.is_contiguous():
            raise ValueError("libkalm takes contiguous tensors")


def version() -> int:
    return load().kalm_version()


def device_check() -> int:
    return load().kalm_device_check()


def kalm_pair_layout(lq: torch.Tensor, n_docs: int, rows: Optional[int] = None, with_h0_row: bool = True,
                     stream=None):
    """lq [Q] int32 (device) -> dict(cu_q, doc_of_pair, final_row, h0_row, h0_final, cu_u)."""
    _contig(lq)
    Qn = lq.numel()
    P = Qn * n_docs
    dev = lq.device
    cu_q = torch.empty(P + 1, dtype=torch.int32, device=dev)
    doc = torch.empty(P, dtype=torch.int32, device=dev)
    fin = torch.empty(P, dtype=torch.int32, device=dev)
    h0 = None
    if with_h0_row:
        if rows is None:
            raise ValueError("rows (= n_docs * sum(lq)) is needed for h0_row")
        h0 = torch.empty(rows, dtype=torch.int32, device=dev)
    h0f = torch.empty(P, dtype=torch.int32, device=dev)
    cu_u = torch.empty(Qn + 1, dtype=torch.int32, device=dev)
    _check("kalm_pair_layout", load().kalm_pair_layout(_ptr(lq), Qn, n_docs, _ptr(cu_q), _ptr(doc), _ptr(fin),
                                                      _ptr(h0), rows or 0, _ptr(h0f), _ptr(cu_u), _stream(stream)))
    return dict(cu_q=cu_q, doc_of_pair=doc, final_row=fin, h0_row=h0, h0_final=h0f, cu_u=cu_u)


def kalm_chunk_pool(x: torch.Tensor, token_mask: torch.Tensor, chunk: int = 4, out=None, stream=None):
    """x [D,T,H] (bf16/f32), token_mask [D,T] uint8 -> (pooled [D,C,H], chunk_mask [D,C], n_chunks [D])."""
    _contig(x, token_mask)
    D, T, H = x.shape
    C = -(-T // chunk)
    if out is None:
        out = (torch.empty(D, C, H, dtype=x.dtype, device=x.device),
               torch.empty(D, C, dtype=torch.uint8, device=x.device),
               torch.empty(D, dtype=torch.int32, device=x.device))
    pooled, cm, nc = out
    _check("kalm_chunk_pool", load().kalm_chunk_pool(_ptr(x), _ptr(token_mask), D, T, H, chunk, _dt(x), _ptr(pooled),
                                                    _ptr(cm), _ptr(nc), _stream(stream)))
    return pooled, cm, nc


def kalm_cross_kv(pooled: torch.Tensor, chunk_mask: Optional[torch.Tensor], Wkv: torch.Tensor, out=None,
                  stream=None):
    """pooled [D,C,H], Wkv [2*kv_dim,H] -> KVc [D,C,2*kv_dim] (keys then values per row)."""
    _contig(pooled, chunk_mask, Wkv)
    D, C, H = pooled.shape
    kv_dim = Wkv.shape[0] // 2
    if out is None:
        out = torch.empty(D, C, 2 * kv_dim, dtype=pooled.dtype, device=pooled.device)
    _check("kalm_cross_kv", load().kalm_cross_kv(_ptr(pooled), _ptr(chunk_mask), D, C, H, _ptr(Wkv), kv_dim,
                                                _dt(pooled), _ptr(out), _stream(stream)))
    return out


def kalm_cross_kv_layers(pooled: torch.Tensor, chunk_mask: Optional[torch.Tensor], Wkv: torch.Tensor, out=None,
                         stream=None):
    """pooled [D,C,H], Wkv [L,2*kv_dim,H] -> KVc [D,C,L,2*kv_dim] (every layer's keys then values per row,
    one launch)."""
    _contig(pooled, chunk_mask, Wkv)
    D, C, H = pooled.shape
    L, two_kv, _ = Wkv.shape
    kv_dim = two_kv // 2
    if out is None:
        out = torch.empty(D, C, L, 2 * kv_dim, dtype=pooled.dtype, device=pooled.device)
    _check("kalm_cross_kv_layers", load().kalm_cross_kv_layers(
        _ptr(pooled), _ptr(chunk_mask), D, C, H, _ptr(Wkv), kv_dim, L, _dt(pooled), _ptr(out), _stream(stream)))
    return out


def kalm_merged_attn(Q: torch.Tensor, Ks: torch.Tensor, Vs: torch.Tensor, cu_q: torch.Tensor, max_lq: int,
                     Kc: torch.Tensor, Vc: torch.Tensor, chunk_mask: torch.Tensor, doc_of_pair: torch.Tensor,
                     nq: int, nkv: int, d: int, scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                     lse: Optional[torch.Tensor] = None, stream=None):
    """Q [rows, >=nq*d] (row stride Q.stride(0)), Ks/Vs [rows, >=nkv*d], Kc/Vc [D*Cmax, >=nkv*d]
    (row-strided views allowed, unit column stride) -> O [rows, nq*d]."""
    for t in (Q, Ks, Vs, Kc, Vc):
        if t.stride(-1) != 1:
            raise ValueError("unit column stride required")
    rows = Q.shape[0]
    P = cu_q.numel() - 1
    D, Cmax = chunk_mask.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty(rows, nq * d, dtype=Q.dtype, device=Q.device)
    _check("kalm_merged_attn", load().kalm_merged_attn(
        _ptr(Q), Q.stride(0), _ptr(Ks), _ptr(Vs), Ks.stride(0), _ptr(cu_q), P, rows, max_lq,
        _ptr(Kc), _ptr(Vc), Kc.stride(0), _ptr(chunk_mask), _ptr(doc_of_pair), D, Cmax, nq, nkv, d,
        float(scale), _dt(Q), _ptr(out), out.stride(0), _ptr(lse), _stream(stream)))
    return out


ROWS_ALL, ROWS_FINAL, ROWS_SHARED, ROWS_SHARED_FINAL = 0, 1, 2, 3


def kalm_merged_attn_rows(Q: torch.Tensor, Ks: torch.Tensor, Vs: torch.Tensor, cu_q: torch.Tensor, max_lq: int,
                          Kc: torch.Tensor, Vc: torch.Tensor, chunk_mask: torch.Tensor, doc_of_pair: torch.Tensor,
                          nq: int, nkv: int, d: int, row_mode: int, o_rows: int, scale: Optional[float] = None,
                          out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None, stream=None):
    """Merged attention over a choice of query rows (row_mode ROWS_ALL / ROWS_FINAL / ROWS_SHARED):
    Q [q_rows, >=nq*d], Ks/Vs [kv_rows, >=nkv*d] -> O [o_rows, nq*d]."""
    for t in (Q, Ks, Vs, Kc, Vc):
        if t.stride(-1) != 1:
            raise ValueError("unit column stride required")
    P = cu_q.numel() - 1
    D, Cmax = chunk_mask.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty(o_rows, nq * d, dtype=Q.dtype, device=Q.device)
    _check("kalm_merged_attn_rows", load().kalm_merged_attn_rows(
        _ptr(Q), Q.stride(0), Q.shape[0], _ptr(Ks), _ptr(Vs), Ks.stride(0), Ks.shape[0], _ptr(cu_q), P, max_lq,
        _ptr(Kc), _ptr(Vc), Kc.stride(0), _ptr(chunk_mask), _ptr(doc_of_pair), D, Cmax, nq, nkv, d,
        float(scale), _dt(Q), _ptr(out), out.stride(0), o_rows, _ptr(lse), int(row_mode), _stream(stream)))
    return out


def kalm_self_attn_partial(Q: torch.Tensor, Ks: torch.Tensor, Vs: torch.Tensor, cu_s: torch.Tensor, max_len: int,
                           nq: int, nkv: int, d: int, scale: Optional[float] = None,
                           out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None, stream=None):
    """Causal self-attention of packed sequences (rows cu_s[i] .. cu_s[i+1]-1):
    Q [rows, >=nq*d], Ks/Vs [rows, >=nkv*d] -> (O [rows, nq*d] float32, lse [rows, nq] float32)."""
    for t in (Q, Ks, Vs):
        if t.stride(-1) != 1:
            raise ValueError("unit column stride required")
    rows = Q.shape[0]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty(rows, nq * d, dtype=torch.float32, device=Q.device)
    if lse is None:
        lse = torch.empty(rows, nq, dtype=torch.float32, device=Q.device)
    _check("kalm_self_attn_partial", load().kalm_self_attn_partial(
        _ptr(Q), Q.stride(0), _ptr(Ks), _ptr(Vs), Ks.stride(0), rows, _ptr(cu_s), cu_s.numel() - 1, max_len, nq, nkv,
        d, float(scale), _dt(Q), _ptr(out), out.stride(0), _ptr(lse), _stream(stream)))
    return out, lse


def kalm_merged_attn_resume(Q: torch.Tensor, o_self: torch.Tensor, lse_self: torch.Tensor, cu_q: torch.Tensor,
                            max_lq: int, Kc: torch.Tensor, Vc: torch.Tensor, chunk_mask: torch.Tensor,
                            doc_of_pair: torch.Tensor, nq: int, nkv: int, d: int, row_mode: int, o_rows: int,
                            scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                            lse: Optional[torch.Tensor] = None, stream=None):
    """Merged attention finished from a self partial (o_self, lse_self indexed like the Q rows):
    only the cross keys are read.  Rows as kalm_merged_attn_rows -> O [o_rows, nq*d]."""
    for t in (Q, o_self, Kc, Vc):
        if t.stride(-1) != 1:
            raise ValueError("unit column stride required")
    _contig(lse_self)
    P = cu_q.numel() - 1
    D, Cmax = chunk_mask.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty(o_rows, nq * d, dtype=Q.dtype, device=Q.device)
    _check("kalm_merged_attn_resume", load().kalm_merged_attn_resume(
        _ptr(Q), Q.stride(0), Q.shape[0], _ptr(o_self), o_self.stride(0), _ptr(lse_self), _ptr(cu_q), P, max_lq,
        _ptr(Kc), _ptr(Vc), Kc.stride(0), _ptr(chunk_mask), _ptr(doc_of_pair), D, Cmax, nq, nkv, d, float(scale),
        _dt(Q), _ptr(out), out.stride(0), o_rows, _ptr(lse), int(row_mode), _stream(stream)))
    return out


def split_workspace_bytes(n_split: int, o_rows: int, nq: int, d: int) -> int:
    """Bytes of workspace kalm_merged_attn_split needs."""
    return n_split * o_rows * nq * (d + 1) * 4


def kalm_merged_attn_split(Q: torch.Tensor, o_self: torch.Tensor, lse_self: torch.Tensor, cu_q: torch.Tensor,
                           max_lq: int, Kc: torch.Tensor, Vc: torch.Tensor, chunk_mask: torch.Tensor,
                           doc_of_pair: torch.Tensor, nq: int, nkv: int, d: int, row_mode: int, o_rows: int,
                           n_split: int, workspace: Optional[torch.Tensor] = None, scale: Optional[float] = None,
                           out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None, stream=None):
    """kalm_merged_attn_resume with the cross keys in n_split shares (split-KV), merged by
    log-sum-exp weights; ``workspace`` (uint8 or any dtype, >= split_workspace_bytes) is
    allocated here when not given."""
    for t in (Q, o_self, Kc, Vc):
        if t.stride(-1) != 1:
            raise ValueError("unit column stride required")
    _contig(lse_self, workspace)
    P = cu_q.numel() - 1
    D, Cmax = chunk_mask.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty(o_rows, nq * d, dtype=Q.dtype, device=Q.device)
    need = split_workspace_bytes(n_split, o_rows, nq, d)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=Q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check("kalm_merged_attn_split", load().kalm_merged_attn_split(
        _ptr(Q), Q.stride(0), Q.shape[0], _ptr(o_self), o_self.stride(0), _ptr(lse_self), _ptr(cu_q), P, max_lq,
        _ptr(Kc), _ptr(Vc), Kc.stride(0), _ptr(chunk_mask), _ptr(doc_of_pair), D, Cmax, nq, nkv, d, float(scale),
        _dt(Q), _ptr(out), out.stride(0), o_rows, _ptr(lse), int(row_mode), int(n_split), _ptr(workspace), ws_bytes,
        _stream(stream)))
    return out


NOALLOC_SCRATCH_BYTES = 16 << 20  # the static split-KV scratch of kalm_merged_attn_split_noalloc


def kalm_merged_attn_split_noalloc(Q: torch.Tensor, o_self: torch.Tensor, lse_self: torch.Tensor,
                                   cu_q: torch.Tensor, max_lq: int, Kc: torch.Tensor, Vc: torch.Tensor,
                                   chunk_mask: torch.Tensor, doc_of_pair: torch.Tensor, nq: int, nkv: int, d: int,
                                   row_mode: int, o_rows: int, n_split: int, out: torch.Tensor,
                                   scale: Optional[float] = None, lse: Optional[torch.Tensor] = None, stream=None):
    """kalm_merged_attn_split with the split partials in the library's static device scratch
    (no workspace, nothing allocated by the call; ``out`` is required).  Calls that overlap on
    one GPU race on the scratch."""
    for t in (Q, o_self, Kc, Vc):
        if t.stride(-1) != 1:
            raise ValueError("unit column stride required")
    _contig(lse_self)
    P = cu_q.numel() - 1
    D, Cmax = chunk_mask.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _check("kalm_merged_attn_split_noalloc", load().kalm_merged_attn_split_noalloc(
        _ptr(Q), Q.stride(0), Q.shape[0], _ptr(o_self), o_self.stride(0), _ptr(lse_self), _ptr(cu_q), P, max_lq,
        _ptr(Kc), _ptr(Vc), Kc.stride(0), _ptr(chunk_mask), _ptr(doc_of_pair), D, Cmax, nq, nkv, d, float(scale),
        _dt(Q), _ptr(out), out.stride(0), o_rows, _ptr(lse), int(row_mode), int(n_split), _stream(stream)))
    return out


def kalm_rms_norm(x: torch.Tensor, w: torch.Tensor, eps: float = 1e-6, out: Optional[torch.Tensor] = None,
                  y_dtype: Optional[torch.dtype] = None, stream=None):
    """y = x / sqrt(mean(x^2) + eps) * w row by row; x [M, H] (row stride >= H), w [H]."""
    if x.stride(-1) != 1:
        raise ValueError("unit column stride required")
    _contig(w)
    M, H = x.shape
    if out is None:
        out = torch.empty(M, H, dtype=y_dtype or x.dtype, device=x.device)
    _check("kalm_rms_norm", load().kalm_rms_norm(_ptr(x), _dt(x), x.stride(0), M, H, _ptr(w), _dt(w), float(eps),
                                                _ptr(out), _dt(out), out.stride(0), _stream(stream)))
    return out


def kalm_rope(X: torch.Tensor, col0: int, n_heads: int, d: int, cu: torch.Tensor, max_len: int, row_mode: int = 0,
              theta: float = 10000.0, stream=None):
    """Rotary embedding in place on heads [col0, col0 + n_heads*d) of X [rows, ld]."""
    if X.stride(-1) != 1:
        raise ValueError("unit column stride required")
    _contig(cu)
    _check("kalm_rope", load().kalm_rope(_ptr(X), _dt(X), X.stride(0), X.shape[0], col0, n_heads, d, _ptr(cu),
                                        cu.numel() - 1, max_len, int(row_mode), float(theta), _stream(stream)))
    return X


def kalm_gated_gelu(Y: torch.Tensor, out: Optional[torch.Tensor] = None, stream=None):
    """Y [M, 2I] (gate | up) -> gelu_tanh(gate) * up [M, I]."""
    if Y.stride(-1) != 1:
        raise ValueError("unit column stride required")
    M, I2 = Y.shape
    I = I2 // 2
    if out is None:
        out = torch.empty(M, I, dtype=Y.dtype, device=Y.device)
    _check("kalm_gated_gelu", load().kalm_gated_gelu(_ptr(Y), _dt(Y), Y.stride(0), M, I, _ptr(out), out.stride(0),
                                                    _stream(stream)))
    return out


def kalm_linear_gated_gelu(X: torch.Tensor, Wg: torch.Tensor, Wu: torch.Tensor, out: Optional[torch.Tensor] = None,
                           stream=None):
    """X [M, K], Wg, Wu [I, K] (bf16) -> gelu_tanh(X Wg^T) * (X Wu^T) [M, I] bf16, fused."""
    _contig(X, Wg, Wu, out)
    M, K = X.shape
    I = Wg.shape[0]
    if Wu.shape != Wg.shape or Wg.shape[1] != K:
        raise ValueError("Wg and Wu must both be [I, K]")
    if out is None:
        out = torch.empty(M, I, dtype=X.dtype, device=X.device)
    _check("kalm_linear_gated_gelu", load().kalm_linear_gated_gelu(_ptr(X), _ptr(Wg), _ptr(Wu), M, K, I, _ptr(out),
                                                                  _stream(stream)))
    return out


def kalm_yesno_score(h: torch.Tensor, final_row: torch.Tensor, w_yesno: torch.Tensor, stream=None):
    """h [rows,H] (f32/bf16), final_row [P], w_yesno [2,H] -> (yes, no, margin, score) [P] float32."""
    P = final_row.numel()
    H = h.shape[1]
    outs = [torch.empty(P, dtype=torch.float32, device=h.device) for _ in range(4)]
    _check("kalm_yesno_score", load().kalm_yesno_score(_ptr(h), _dt(h), h.stride(0), h.shape[0], _ptr(final_row), P, H,
                                                      _ptr(w_yesno), _dt(w_yesno), *[_ptr(o) for o in outs],
                                                      _stream(stream)))
    return tuple(outs)


def kalm_linear(X: torch.Tensor, W: torch.Tensor, Y: Optional[torch.Tensor] = None, accumulate: bool = False,
                y_dtype: Optional[torch.dtype] = None, Y_bf16: Optional[torch.Tensor] = None, stream=None):
    """Y = X W^T (or Y += X W^T for an fp32 Y); optional bf16 copy of the result."""
    _contig(X, W, Y, Y_bf16)
    M, K = X.shape
    N = W.shape[0]
    if Y is None:
        Y = torch.empty(M, N, dtype=y_dtype or X.dtype, device=X.device)
    _check("kalm_linear", load().kalm_linear(_ptr(X), _ptr(W), M, K, N, _dt(X), _ptr(Y), _dt(Y),
                                            1 if accumulate else 0, _ptr(Y_bf16), _stream(stream)))
    return Y


def kalm_linear_residual(X: torch.Tensor, W: torch.Tensor, R: torch.Tensor, r_row: Optional[torch.Tensor],
                         Y: Optional[torch.Tensor] = None, Y_bf16: Optional[torch.Tensor] = None, stream=None):
    """Y = R[r_row] + X W^T (fp32; R row m when r_row is None); optional bf16 copy."""
    _contig(X, W, R, r_row, Y, Y_bf16)
    M, K = X.shape
    N = W.shape[0]
    if Y is None:
        Y = torch.empty(M, N, dtype=torch.float32, device=X.device)
    _check("kalm_linear_residual", load().kalm_linear_residual(
        _ptr(X), _ptr(W), M, K, N, _dt(X), _ptr(R), _ptr(r_row), R.shape[0], _ptr(Y), _ptr(Y_bf16),
        _stream(stream)))
    return Y


def kalm_gather_rows(src: torch.Tensor, idx: torch.Tensor, dst: Optional[torch.Tensor] = None,
                     dst_bf16: Optional[torch.Tensor] = None, stream=None):
    _contig(src, idx, dst, dst_bf16)
    n_src, H = src.shape
    M = idx.numel()
    if dst is None:
        dst = torch.empty(M, H, dtype=torch.float32, device=src.device)
    _check("kalm_gather_rows", load().kalm_gather_rows(_ptr(src), _ptr(idx), M, H, n_src, _ptr(dst), _ptr(dst_bf16),
                                                      _stream(stream)))
    return dst


def kalm_rank_topn(score: torch.Tensor, top_n: int, stream=None):
    """score [Q, D] float32 -> (index [Q, top_n] int32, score [Q, top_n] float32), best first."""
    _contig(score)
    Qn, D = score.shape
    idx = torch.empty(Qn, top_n, dtype=torch.int32, device=score.device)
    val = torch.empty(Qn, top_n, dtype=torch.float32, device=score.device)
    _check("kalm_rank_topn", load().kalm_rank_topn(_ptr(score), Qn, D, top_n, _ptr(idx), _ptr(val),
                                                  _stream(stream)))
    return idx, val

