"""The C-ABI library loads and exports every function include/biverify.h
declares; host-side argument checks reject bad calls without launching (CPU
only: no compute call reaches the GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "biverify.h")
LIB = os.path.join(ROOT, "invariant_verify_verifier_amd", "libbiverify.so")


def declared_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    names = re.findall(r"^(?:biv_status|int|size_t|const char\*)\s+(\w+)\s*\(", txt, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_five_hot_path_calls():
    names = declared_functions()
    for n in ["rmsnorm_bi", "gemm_bi", "attn_decode_bi", "gumbel_verify", "kv_overwrite"]:
        assert n in names


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail(f"{LIB} not built (run __graft_entry__.build())")
    return ctypes.CDLL(LIB)


def test_library_exports_every_declared_symbol(lib):
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_binding_covers_every_declared_symbol():
    import invariant_verify_verifier_amd as m

    assert sorted(m.exported_symbols()) == declared_functions()


def test_host_side_argument_errors(lib):
    """Bad sizes, dtypes and NULL pointers return BIV_EINVAL before any launch."""
    lib.biv_last_error.restype = ctypes.c_char_p
    vp, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
    lib.gemm_bi.argtypes = [vp, vp, vp, i64, i64, i64, i32, i32, i32, vp]
    assert lib.gemm_bi(None, None, None, 4, 8, 8, 1, 1, 0, None) == 1  # NULL pointers
    assert b"NULL" in lib.biv_last_error()
    assert lib.gemm_bi(None, None, None, 4, 8, 8, 7, 1, 0, None) == 1  # bad dtype
    assert lib.gemm_bi(None, None, None, 0, 8, 8, 1, 1, 0, None) == 0  # M = 0: nothing to do
    buf = ctypes.create_string_buffer(4096)
    bp = ctypes.cast(buf, vp)
    assert lib.gemm_bi(bp, bp, bp, 4, 128, 96, 1, 1, 2, None) == 1  # SwiGLU epilogue: K % 64 != 0
    assert lib.gemm_bi(bp, bp, bp, 4, 96, 64, 1, 1, 2, None) == 1  # SwiGLU epilogue: N % 64 != 0
    assert lib.gemm_bi(bp, bp, bp, 4, 128, 64, 0, 0, 2, None) == 1  # SwiGLU epilogue: fp32 inputs
    assert lib.gemm_bi(bp, bp, bp, 4, 128, 64, 1, 1, 3, None) == 1  # unknown epilogue
    lib.rmsnorm_bi.argtypes = [vp, i32, vp, vp, vp, i32, i64, i64, f32, vp]
    assert lib.rmsnorm_bi(None, 0, None, None, None, 0, 3, 0, 1e-6, None) == 1  # H = 0
    assert lib.rmsnorm_bi(None, 0, None, None, None, 0, 0, 8, 1e-6, None) == 0  # M = 0: nothing to do
    big = ctypes.create_string_buffer(1 << 16)
    b0 = ctypes.cast(big, vp).value
    # x and y overlap; residual overlapping x (4 rows of 64 fp32 = 1 KiB each)
    assert lib.rmsnorm_bi(b0, 0, None, b0 + 8192, b0 + 512, 0, 4, 64, 1e-6, None) == 1
    assert b"overlap" in lib.biv_last_error()
    assert lib.rmsnorm_bi(b0, 0, b0 + 512, b0 + 8192, b0 + 16384, 0, 4, 64, 1e-6, None) == 1
    assert b"overlap" in lib.biv_last_error()
    lib.gumbel_verify.argtypes = [vp, vp, vp, i32, i32, i32, vp, vp, vp, vp]
    assert lib.gumbel_verify(None, None, None, 2, 0, 8, None, None, None, None) == 1  # K = 0
    assert lib.gumbel_verify(None, None, None, 0, 4, 8, None, None, None, None) == 0  # R = 0
    lib.kv_overwrite.argtypes = [vp, vp, i64, vp, vp, vp, i32, i32, i32, i32, i32, vp]
    assert lib.kv_overwrite(None, None, 4, None, None, None, 1, 8, 128, 10, 1, None) == 1  # stride < Hkv*D
    lib.gumbel_topk.argtypes = [vp, vp, i32, i32, i32, vp, vp, vp]
    assert lib.gumbel_topk(bp, bp, 4, 100, 9, bp, None, None) == 2  # k > 8: unsupported
    assert lib.gumbel_topk(bp, bp, 4, 5, 6, bp, None, None) == 1  # k > V
    assert lib.gumbel_topk(None, None, 0, 100, 3, None, None, None) == 0  # no rows
    lib.lm_head_gumbel_verify.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.biv_gumbel_workspace_bytes.argtypes = [i32, i32]
    lib.biv_gumbel_workspace_bytes.restype = ctypes.c_size_t
    assert lib.biv_gumbel_workspace_bytes(512, 128256) == 512 * 2004 * 8
    assert lib.biv_gumbel_workspace_bytes(3, 65) == 3 * 2 * 8
    # H not a multiple of 64
    assert lib.lm_head_gumbel_verify(bp, bp, bp, bp, 2, 4, 1000, 100, bp, bp, bp, bp, 1 << 20, None) == 1
    # workspace too small
    assert lib.lm_head_gumbel_verify(bp, bp, bp, bp, 2, 4, 1000, 128, bp, bp, bp, bp, 8, None) == 1
    assert b"workspace" in lib.biv_last_error()
    assert lib.lm_head_gumbel_verify(None, None, None, None, 0, 4, 1000, 128, None, None, None, None, 0, None) == 0
    lib.rope_kv_overwrite.argtypes = [vp, i64, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, vp]
    # stride < (Hq + 2*Hkv) * D
    assert lib.rope_kv_overwrite(bp, 6000, bp, bp, bp, bp, bp, 1, 32, 8, 128, 16, 4, 1, None) == 1
    assert lib.rope_kv_overwrite(bp, 6144, bp, bp, bp, bp, bp, 1, 32, 8, 127, 16, 4, 1, None) == 1  # odd D
    assert lib.rope_kv_overwrite(None, 6144, None, None, None, None, None, 0, 32, 8, 128, 16, 4, 1, None) == 0
    lib.attn_decode_bi.argtypes = [vp, i64, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32, i32, vp,
                                   ctypes.c_size_t, vp]
    # Hq not a multiple of Hkv
    assert lib.attn_decode_bi(None, 4096, None, None, None, None, None, None, 1, 1, 30, 8, 128, 4, 4, 0.1, 1, None, 0,
                              None) == 1
    # bf16 path: G = Hq/Hkv must divide 32 (unsupported otherwise, not invalid); q_len * G > 32 takes
    # several row blocks and a workspace sized for them
    buf = ctypes.create_string_buffer(64)
    p = ctypes.cast(buf, vp)
    assert lib.attn_decode_bi(p, 4096, p, p, p, p, None, p, 1, 16, 24, 8, 128, 4, 4, 0.1, 1, p, 64, None) == 2
    assert lib.attn_decode_bi(p, 4096, p, p, p, p, None, p, 1, 16, 32, 8, 128, 4, 4, 0.1, 1, p, 64, None) == 1
    assert b"workspace" in lib.biv_last_error()
    # with row offsets the workspace is sized by q_len, the most rows of any request
    assert lib.attn_decode_bi(p, 4096, p, p, p, p, p, p, 2, 16, 32, 8, 128, 4, 4, 0.1, 1, p, 64, None) == 1
    assert b"workspace" in lib.biv_last_error()
    assert lib.attn_decode_bi(p, 4096, p, p, p, p, p, p, 0, 16, 32, 8, 128, 4, 4, 0.1, 1, None, 0, None) == 0
    lib.biv_attn_workspace_bytes_q.restype = ctypes.c_size_t
    lib.biv_attn_workspace_bytes_q.argtypes = [ctypes.c_int] * 6
    lib.biv_attn_workspace_bytes.restype = ctypes.c_size_t
    lib.biv_attn_workspace_bytes.argtypes = [ctypes.c_int] * 4
    # 200 rows, G = 4: 25 row blocks of 8 positions
    assert lib.biv_attn_workspace_bytes_q(3, 200, 32, 8, 40, 2048) == lib.biv_attn_workspace_bytes(75, 8, 40, 2048)
    assert lib.biv_attn_workspace_bytes_q(3, 8, 32, 8, 40, 2048) == lib.biv_attn_workspace_bytes(3, 8, 40, 2048)
    assert lib.biv_attn_workspace_bytes_q(3, 8, 24, 8, 40, 2048) == 0


def test_abi_version(lib):
    lib.biv_abi_version.restype = ctypes.c_int
    assert lib.biv_abi_version() == 2


def test_workspace_sizes(lib):
    lib.biv_attn_workspace_bytes.restype = ctypes.c_size_t
    lib.biv_attn_workspace_bytes.argtypes = [ctypes.c_int] * 4
    n = lib.biv_attn_workspace_bytes(64, 8, 513, 1024)
    nseg = -(-513 * 16 // 1024)
    assert n == 64 * 8 * nseg * (4096 + 128) * 4 + 64 * nseg * 4  # segment results + work list
    # one request, contexts up to 32768: its 8 x 8 segment waves are split 16
    # ways (one 256-token chunk each), with room for every chunk's partial
    n1 = lib.biv_attn_workspace_bytes(1, 8, 2048, 4096)
    assert n1 == (8 * 8 + 8 * 8 * 16) * (4096 + 128) * 4 + 8 * 4
    # the comparison path's splits are multiples of 256 tokens
    assert lib.biv_attn_workspace_bytes(1, 8, 2048, 256) == 8 * 128 * (4096 + 128) * 4 + 128 * 4
    assert lib.biv_attn_workspace_bytes(1, 8, 2048, 200) == 0
    lib.biv_splitk_auto_splits.restype = ctypes.c_int
    lib.biv_splitk_auto_splits.argtypes = [ctypes.c_int64] * 3
    # the staged kernel's own grid: M = 1 on a 14336-wide weight is 224 tiles of
    # 32 x 64 (fewer than 256 CUs) -> 2 splits; M = 512 already fills the GPU -> 1
    assert lib.biv_splitk_auto_splits(1, 14336, 4096) == 2
    assert lib.biv_splitk_auto_splits(1, 4096, 14336) == 4  # 64 tiles
    assert lib.biv_splitk_auto_splits(512, 14336, 4096) == 1
    assert lib.biv_splitk_auto_splits(512, 4096, 4096) == 1  # 256 tiles of 128 x 64
    assert lib.biv_splitk_auto_splits(1, 4096, 512) == 2  # every split keeps >= 4 k stages of 64
    assert lib.biv_splitk_auto_splits(1, 4096, 256) == 1


def test_rope_table_host_values(lib):
    """The library's host RoPE table: pos 3, pair 0 turns by 3 rad; pair i by
    3 * theta^(-2i/D)."""
    import math

    lib.biv_rope_table.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_double]
    D, P = 8, 5
    buf = (ctypes.c_float * (P * D))()
    assert lib.biv_rope_table(ctypes.cast(buf, ctypes.c_void_p), P, D, 100.0) == 0
    for i in range(D // 2):
        a = 3 * 100.0 ** (-2 * i / D)
        assert abs(buf[(3 * D // 2 + i) * 2] - math.cos(a)) < 1e-7
        assert abs(buf[(3 * D // 2 + i) * 2 + 1] - math.sin(a)) < 1e-7


def test_dvr_round_stats_and_rollback_rule():
    """Host bookkeeping of decode-verify-rollback (LLM-42 post, paragraph 3):
    acceptance is the accepted share of drafted tokens, tokens per round the
    committed count (prefix plus correction, all K when nothing diverges)."""
    import numpy as np

    from invariant_verify_verifier_amd import dvr, verifier

    st = dvr.RoundStats()
    assert np.isnan(st.acceptance(8)) and np.isnan(st.tokens_per_round())
    cand = np.array([[5, 6, 7, 8], [5, 6, 7, 8], [5, 6, 7, 8]])
    acc = np.array([0, 2, 4])
    new_ctx, committed, t0 = verifier.rollback(np.array([10, 20, 30]), acc, np.array([9, 9, -1]), cand)
    assert list(new_ctx) == [11, 23, 34] and committed == [[9], [5, 6, 9], [5, 6, 7, 8]] and list(t0) == [9, 9, 8]
    st.accept_len.append(acc)
    st.committed.append(np.array([len(c) for c in committed]))
    assert st.acceptance(4) == 0.5 and abs(st.tokens_per_round() - 8 / 3) < 1e-12


def test_tree_adopt_chain_pages_host_rule():
    """After tree verification a request keeps its selected chain's pages for
    L .. L+K-1 and frees the rest (host bookkeeping; no GPU)."""
    import numpy as np

    from invariant_verify_verifier_amd import verifier as V

    bt = np.array([[0, 1, 2, 3], [4, 5, 6, 7]], np.int32)
    ctx = [20, 35]  # request 0: positions 20..23 on page 1; request 1: 35..38 on page 2
    priv = np.array([[[10, 11], [12, 13]], [[14, 15], [16, 17]]], np.int32)  # [R, B-1, 2]
    nbt, freed = V.adopt_chain_pages(bt, ctx, [2, 0], priv, K=4)
    assert nbt.tolist() == [[0, 12, 2, 3], [4, 5, 6, 7]]
    assert sorted(freed[0]) == [1, 10] and sorted(freed[1]) == [14, 16]
    # a span over two pages (L % 16 + K > 16) moves both
    nbt, freed = V.adopt_chain_pages(bt, [30, 0], [1, 1], priv, K=4)
    assert nbt.tolist() == [[0, 10, 11, 3], [14, 5, 6, 7]]
    assert sorted(freed[0]) == [1, 2, 12, 13] and sorted(freed[1]) == [4, 16]
