"""Host-side checks of the C ABI (no GPU needed, no compute call is made).

The built library must load and export every entry point that include/kalm.h
declares; argument validation must reject bad calls before any launch; and
without a GPU every call must report KALM_ERR_NO_DEVICE instead of falling back
to the CPU.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kalm.h")
LIB = os.path.join(ROOT, "encoder_decoder_document_amd", "libkalm.so")
DEBUG_LIB = os.path.join(ROOT, "encoder_decoder_document_amd", "libkalm_debug.so")
BOTH = [pytest.param(LIB, id="release"), pytest.param(DEBUG_LIB, id="debug")]

needs_lib = pytest.mark.skipif(not os.path.exists(LIB), reason="libkalm.so not built (run __graft_entry__.build())")


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kalm_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_hot_path_calls():
    syms = declared_symbols()
    for s in ("kalm_chunk_pool", "kalm_cross_kv", "kalm_cross_kv_layers", "kalm_merged_attn", "kalm_yesno_score",
              "kalm_linear", "kalm_pair_layout", "kalm_gather_rows", "kalm_last_error", "kalm_version",
              "kalm_device_check"):
        assert s in syms


def declared_params(name):
    """Parameter names of one declaration in the header, in order."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    m = re.search(r"\b" + name + r"\s*\(([^)]*)\)\s*;", text)
    assert m, name
    params = [p.strip() for p in m.group(1).split(",")]
    return [re.findall(r"[A-Za-z_][A-Za-z0-9_]*", p)[-1] for p in params if p and p != "void"]


# The five boundary calls: their planned parameter lists (the names the hot
# path's steps fix), the lists as built, and every departure between them --
# each one is listed with its reason in the design notes.  A change to a
# signature fails here until the departure is recorded.
PLANNED = {
    "kalm_chunk_pool": "x token_mask D T H chunk dt pooled chunk_mask n_chunks s",
    "kalm_cross_kv": "pooled n_chunks D Cmax H Wk Wv kv_dim dt Kc Vc s",
    "kalm_merged_attn": "Q Ks Vs cu_q P Kc Vc chunk_mask doc_of_pair Cmax nq nkv d scale dt O lse s",
    "kalm_yesno_score": "h final_row P H w_yesno w_dt yes no margin score s",
    "kalm_linear": "X x_dt W M K N Y y_dt accumulate_fp32 s",
}
BUILT = {
    "kalm_chunk_pool": "x token_mask D T H chunk dt pooled chunk_mask n_chunks stream",
    "kalm_cross_kv": "pooled chunk_mask D Cmax H Wkv kv_dim dt KVc stream",
    "kalm_merged_attn": "Q q_ld Ks Vs kv_ld cu_q P rows max_lq Kc Vc c_ld chunk_mask doc_of_pair D Cmax nq nkv d "
                        "scale dt O o_ld lse stream",
    "kalm_yesno_score": "h h_dt h_ld rows final_row P H w_yesno w_dt yes no margin score stream",
    "kalm_linear": "X W M K N dt Y y_dt accumulate Y_bf16 stream",
}
# (planned names not kept, built names added)
DEPARTURES = {
    "kalm_chunk_pool": ({"s"}, {"stream"}),
    "kalm_cross_kv": ({"n_chunks", "Wk", "Wv", "Kc", "Vc", "s"}, {"chunk_mask", "Wkv", "KVc", "stream"}),
    "kalm_merged_attn": ({"s"}, {"q_ld", "kv_ld", "rows", "max_lq", "c_ld", "D", "o_ld", "stream"}),
    "kalm_yesno_score": ({"s"}, {"h_dt", "h_ld", "rows", "stream"}),
    "kalm_linear": ({"x_dt", "accumulate_fp32", "s"}, {"dt", "accumulate", "Y_bf16", "stream"}),
}


@pytest.mark.parametrize("name", sorted(PLANNED))
def test_boundary_parameter_lists(name):
    got = declared_params(name)
    assert got == BUILT[name].split(), f"{name}: {got}"
    planned = set(PLANNED[name].split())
    dropped, added = DEPARTURES[name]
    assert planned - set(got) == dropped, f"{name}: undocumented departure {planned - set(got)}"
    assert set(got) - planned == added, f"{name}: undocumented addition {set(got) - planned}"
    # every kept name keeps its relative order
    kept = [p for p in got if p in planned]
    assert kept == [p for p in PLANNED[name].split() if p in set(got)], name


@needs_lib
@pytest.mark.parametrize("path", BOTH)
def test_library_exports_every_declared_symbol(path):
    lib = ctypes.CDLL(path)
    missing = [s for s in declared_symbols() if not hasattr(lib, s)]
    assert not missing, f"not exported: {missing}"


@needs_lib
@pytest.mark.parametrize("path,flag", [(LIB, 0), (DEBUG_LIB, 1)])
def test_debug_build_reports_itself(path, flag):
    # the two builds share every entry point; only the debug one records guards
    lib = ctypes.CDLL(path)
    lib.kalm_debug_build.restype = ctypes.c_int32
    lib.kalm_version.restype = ctypes.c_int32
    assert lib.kalm_debug_build() == flag
    assert lib.kalm_version() == 400


@needs_lib
def test_binding_covers_every_declared_symbol():
    from encoder_decoder_document_amd import ops
    assert sorted(ops.EXPORTED) == declared_symbols()


@needs_lib
@pytest.mark.parametrize("path", BOTH)
def test_invalid_arguments_rejected_before_launch(path):
    from encoder_decoder_document_amd import ops
    lib = ops.load(path)
    assert lib.kalm_version() == 400
    # chunk = 0
    st = lib.kalm_chunk_pool(None, None, 1, 8, 64, 0, ops.KALM_BF16, None, None, None, None)
    assert st == ops.KALM_ERR_INVALID_ARG and b"chunk" in lib.kalm_last_error()
    # H not a multiple of the 16-byte vector
    st = lib.kalm_chunk_pool(None, None, 1, 8, 12, 4, ops.KALM_BF16, None, None, None, None)
    assert st == ops.KALM_ERR_UNSUPPORTED
    # unsupported dtype
    st = lib.kalm_linear(None, None, 4, 8, 8, 7, None, ops.KALM_F32, 0, None, None)
    assert st == ops.KALM_ERR_UNSUPPORTED
    # accumulate into a bf16 Y (fake, never dereferenced pointers: validation fails first)
    st = lib.kalm_linear(16, 32, 4, 8, 8, ops.KALM_BF16, 48, ops.KALM_BF16, 1, None, None)
    assert st == ops.KALM_ERR_UNSUPPORTED
    # bf16 attention with a head dim other than 256
    st = lib.kalm_merged_attn(None, 512, None, None, 128, None, 0, 0, 0, None, None, 128, None, None, 0, 0,
                              4, 1, 128, 0.1, ops.KALM_BF16, None, 512, None, None)
    assert st == ops.KALM_ERR_UNSUPPORTED
    # nq not a multiple of nkv
    st = lib.kalm_merged_attn(None, 1024, None, None, 768, None, 0, 0, 0, None, None, 768, None, None, 0, 0,
                              4, 3, 256, 0.1, ops.KALM_BF16, None, 1024, None, None)
    assert st == ops.KALM_ERR_INVALID_ARG
    # misaligned pointer
    st = lib.kalm_gather_rows(8, 16, 4, 8, 4, 16, None, None)
    assert st == ops.KALM_ERR_INVALID_ARG
    # attention over a choice of rows: unknown row mode; shared rows without passages
    st = lib.kalm_merged_attn_rows(None, 1024, 0, None, None, 512, 0, None, 0, 0, None, None, 512, None, None, 0, 0,
                                   4, 1, 256, 0.1, ops.KALM_BF16, None, 1024, 0, None, 4, None)
    assert st == ops.KALM_ERR_INVALID_ARG and b"row_mode" in lib.kalm_last_error()
    st = lib.kalm_merged_attn_rows(None, 1024, 0, None, None, 512, 0, None, 1, 0, None, None, 512, None, None, 0, 0,
                                   4, 1, 256, 0.1, ops.KALM_BF16, None, 1024, 0, None, 3, None)
    assert st == ops.KALM_ERR_INVALID_ARG and b"D >= 1" in lib.kalm_last_error()
    st = lib.kalm_merged_attn_rows(None, 1024, 0, None, None, 512, 0, None, 1, 0, None, None, 512, None, None, 0, 0,
                                   4, 1, 256, 0.1, ops.KALM_BF16, None, 1024, 0, None, 2, None)
    assert st == ops.KALM_ERR_INVALID_ARG
    # self partial: its lse output is required
    st = lib.kalm_self_attn_partial(1, 1024, 1, 1, 512, 10, 1, 1, 10, 4, 1, 256, 0.1, ops.KALM_BF16, 1, 1024, None,
                                    None)
    assert st == ops.KALM_ERR_INVALID_ARG and b"lse" in lib.kalm_last_error()
    # resume: the self partial is required; row_mode outside 0..3; partial stride smaller than the heads
    st = lib.kalm_merged_attn_resume(1, 1024, 10, None, 1024, None, 1, 1, 10, 1, 1, 512, 1, 1, 1, 8, 4, 1, 256, 0.1,
                                     ops.KALM_BF16, 1, 1024, 10, None, 0, None)
    assert st == ops.KALM_ERR_INVALID_ARG and b"self-partial" in lib.kalm_last_error()
    st = lib.kalm_merged_attn_resume(1, 1024, 10, 1, 1024, 1, 1, 1, 10, 1, 1, 512, 1, 1, 1, 8, 4, 1, 256, 0.1,
                                     ops.KALM_BF16, 1, 1024, 10, None, -1, None)
    assert st == ops.KALM_ERR_INVALID_ARG and b"row_mode" in lib.kalm_last_error()
    st = lib.kalm_merged_attn_resume(1, 1024, 10, 1, 512, 1, 1, 1, 10, 1, 1, 512, 1, 1, 1, 8, 4, 1, 256, 0.1,
                                     ops.KALM_BF16, 1, 1024, 10, None, 0, None)
    assert st == ops.KALM_ERR_INVALID_ARG and b"leading dimension" in lib.kalm_last_error()
    # split-KV: workspace too small; n_split out of range; fp32 not implemented
    args = (1, 1024, 10, 1, 1024, 1, 1, 1, 10, 1, 1, 512, 1, 1, 1, 8, 4, 1, 256, 0.1, ops.KALM_BF16, 1, 1024, 10,
            None, 0)
    need = 2 * 10 * 4 * 257 * 4
    st = lib.kalm_merged_attn_split(*args, 2, 16, need - 1, None)
    assert st == ops.KALM_ERR_INVALID_ARG and b"workspace" in lib.kalm_last_error()
    st = lib.kalm_merged_attn_split(*args, 65, 16, 1 << 30, None)
    assert st == ops.KALM_ERR_INVALID_ARG and b"n_split" in lib.kalm_last_error()
    st = lib.kalm_merged_attn_split(*args[:20], ops.KALM_F32, *args[21:], 2, 16, need, None)
    assert st == ops.KALM_ERR_UNSUPPORTED
    # the no-allocation split: partials larger than its static scratch are refused before any launch
    big = args[:23] + (1 << 20,) + args[24:]
    st = lib.kalm_merged_attn_split_noalloc(*big, 64, None)
    assert st == ops.KALM_ERR_INVALID_ARG and b"static scratch" in lib.kalm_last_error()
    # gathered residual: no source; without an index the source needs M rows
    st = lib.kalm_linear_residual(16, 16, 10, 64, 64, ops.KALM_BF16, None, None, 10, 16, None, None)
    assert st == ops.KALM_ERR_INVALID_ARG and b"residual source" in lib.kalm_last_error()
    st = lib.kalm_linear_residual(16, 16, 10, 64, 64, ops.KALM_BF16, 16, None, 9, 16, None, None)
    assert st == ops.KALM_ERR_INVALID_ARG and b"M rows" in lib.kalm_last_error()
    # ranking: top_n larger than the passages; too many passages for one workgroup
    st = lib.kalm_rank_topn(None, 1, 10, 11, None, None, None)
    assert st == ops.KALM_ERR_INVALID_ARG and b"top_n" in lib.kalm_last_error()
    st = lib.kalm_rank_topn(None, 1, 5000, 10, None, None, None)
    assert st == ops.KALM_ERR_UNSUPPORTED
    # fused gate/up + activation: width not a multiple of 128; K not a multiple of 8; missing up weights
    st = lib.kalm_linear_gated_gelu(16, 16, 16, 10, 64, 100, 16, None)
    assert st == ops.KALM_ERR_UNSUPPORTED and b"I % 128" in lib.kalm_last_error()
    st = lib.kalm_linear_gated_gelu(16, 16, 16, 10, 60, 128, 16, None)
    assert st == ops.KALM_ERR_UNSUPPORTED
    st = lib.kalm_linear_gated_gelu(16, 16, None, 10, 64, 128, 16, None)
    assert st == ops.KALM_ERR_INVALID_ARG and b"null" in lib.kalm_last_error()
    # launch-size limits (fake, never dereferenced pointers): 2^26 or more pooled rows;
    # 2^31 or more attention work items
    st = lib.kalm_chunk_pool(16, 32, 1 << 20, 1024, 64, 4, ops.KALM_BF16, 48, 64, 80, None)
    assert st == ops.KALM_ERR_UNSUPPORTED and b"2^26" in lib.kalm_last_error()
    st = lib.kalm_merged_attn(16, 1024, 32, 48, 256, 64, 1 << 28, 1 << 30, 512, 80, 96, 256, 112, 128, 1, 4,
                              4, 1, 256, 0.0625, ops.KALM_BF16, 144, 1024, None, None)
    assert st == ops.KALM_ERR_UNSUPPORTED and b"work items" in lib.kalm_last_error()


@needs_lib
@pytest.mark.parametrize("path", BOTH)
def test_no_device_means_error_not_cpu_fallback(path):
    import subprocess
    import sys
    code = (
        "import ctypes,sys; lib=ctypes.CDLL(sys.argv[1]);"
        "lib.kalm_device_check.restype=ctypes.c_int; lib.kalm_last_error.restype=ctypes.c_char_p;"
        "s=lib.kalm_device_check(); print(s, lib.kalm_last_error().decode())"
    )
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1", CUDA_VISIBLE_DEVICES="-1")
    out = subprocess.run([sys.executable, "-c", code, path], capture_output=True, text=True, env=env, timeout=120)
    status = int(out.stdout.split()[0])
    assert status == 3, out.stdout + out.stderr   # KALM_ERR_NO_DEVICE
    assert "no HIP device" in out.stdout or "gfx950" in out.stdout
