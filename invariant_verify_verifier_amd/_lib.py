"""ctypes binding of libbiverify (the C ABI in include/biverify.h).

Argument marshalling only: every function here takes torch tensors that
already live on the GPU, passes their addresses, sizes and torch's current
HIP stream to the library, and raises on a non-OK status.  No computation
happens in Python and there is no fallback: if the library is missing the
import fails loudly.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbiverify.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build the HIP library first "
        "(python -m invariant_verify_verifier_amd.build, or __graft_entry__.build())")

_lib = ctypes.CDLL(LIB_PATH)

BIV_OK, BIV_EINVAL, BIV_EUNSUPPORTED, BIV_EHIP = 0, 1, 2, 3
BIV_F32, BIV_BF16 = 0, 1
BIV_EPI_STORE, BIV_EPI_ACCUM, BIV_EPI_SWIGLU = 0, 1, 2
ATTN_CHUNK_TOKENS = 256
ATTN_SEG_TOKENS = 4096

_vp, _i32, _i64, _f32, _f64, _sz = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float,
                                    ctypes.c_double, ctypes.c_size_t)

_SIGS = {
    "biv_abi_version": ([], _i32),
    "biv_last_error": ([], ctypes.c_char_p),
    "rmsnorm_bi": ([_vp, _i32, _vp, _vp, _vp, _i32, _i64, _i64, _f32, _vp], _i32),
    "gemm_bi": ([_vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _i32, _vp], _i32),
    "biv_attn_workspace_bytes": ([_i32, _i32, _i32, _i32], _sz),
    "biv_attn_workspace_bytes_q": ([_i32, _i32, _i32, _i32, _i32, _i32], _sz),
    "attn_decode_bi": ([_vp, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32,
                        _i32, _vp, _sz, _vp], _i32),
    "attn_decode_bi_static": ([_vp, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                               _f32, _i32, _vp], _i32),
    "gumbel_verify": ([_vp, _vp, _vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp], _i32),
    "gumbel_topk": ([_vp, _vp, _i32, _i32, _i32, _vp, _vp, _vp], _i32),
    "biv_gumbel_workspace_bytes": ([_i32, _i32], _sz),
    "lm_head_gumbel_verify": ([_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _sz, _vp], _i32),
    "kv_overwrite": ([_vp, _vp, _i64, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _vp], _i32),
    "kv_copy_pages": ([_vp, _vp, _i32, _vp, _vp, _i32, _i32, _i32, _i32, _vp], _i32),
    "tree_select": ([_vp, _vp, _i32, _i32, _vp, _vp, _vp, _vp], _i32),
    "embed_rows": ([_vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32, _vp], _i32),
    "biv_rope_table": ([_vp, _i32, _i32, _f64], _i32),
    "rope_apply": ([_vp, _i64, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _vp], _i32),
    "rope_kv_overwrite": ([_vp, _i64, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _vp], _i32),
    "swiglu": ([_vp, _vp, _i64, _i64, _i64, _i32, _vp], _i32),
    "biv_splitk_workspace_bytes": ([_i64, _i64, _i32], _sz),
    "biv_splitk_auto_splits": ([_i64, _i64, _i64], _i32),
    "gemm_splitk": ([_vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _i32, _vp, _sz, _vp], _i32),
    "biv_attn_adaptive_split": ([_i32, _i32, _i32], _i32),
    "attn_decode_adaptive": ([_vp, _i64, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32,
                              _vp, _sz, _vp], _i32),
}

for _name, (_args, _ret) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.argtypes = _args
    _fn.restype = _ret


class BivError(RuntimeError):
    def __init__(self, fn, status):
        msg = _lib.biv_last_error().decode(errors="replace")
        super().__init__(f"{fn}: status {status}: {msg}")
        self.status = status


def _check(fn, status):
    if status != BIV_OK:
        raise BivError(fn, status)


def exported_symbols():
    """Names of the C entry points this binding declares."""
    return list(_SIGS)


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BIV_BF16
    if t.dtype == torch.float32:
        return BIV_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _p(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    return ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _contig(*ts):
    for t in ts:
        if t is not None and not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _same_dtype(*ts):
    d = {t.dtype for t in ts if t is not None}
    if len(d) != 1:
        raise TypeError(f"dtype mismatch: {d}")


def _require(cond, what):
    """Shape/argument check that stays on under ``python -O`` (unlike assert)."""
    if not cond:
        raise ValueError(f"bad argument: {what}")


def _want(t, dtype, name):
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


# ----------------------------------------------------------------- entry points


def rmsnorm_bi(x, gamma, y, eps, residual=None):
    """y = rmsnorm(x) (x [M, H]; gamma [H] and y in one dtype); with
    ``residual`` ([M, H], x's dtype) the row normalised is s = x + residual,
    and s is written back to residual."""
    _contig(x, gamma, y, residual)
    _same_dtype(gamma, y)
    M, H = x.shape
    _require(tuple(y.shape) == (M, H) and gamma.numel() == H, "rmsnorm_bi: y [M, H], gamma [H]")
    if residual is not None:
        _same_dtype(x, residual)
        _require(tuple(residual.shape) == (M, H), "rmsnorm_bi: residual [M, H]")
    _check("rmsnorm_bi", _lib.rmsnorm_bi(_p(x), _dt(x), _p(residual), _p(gamma), _p(y), _dt(y), M, H, eps,
                                         _stream()))
    return y


def gemm_bi(a, b, c, accumulate=False, swiglu=False):
    """c[M,N] (=|+=) a[M,K] @ b[N,K]^T; with swiglu, b is the 32-row-block
    interleaved gate/up weight (pack_gate_up) and c[M, N/2] = silu(gate) * up."""
    _contig(a, b, c)
    M, K = a.shape
    N = b.shape[0]
    _require(b.shape[1] == K, 'b.shape[1] == K')
    _require(tuple(c.shape) == ((M, N // 2) if swiglu else (M, N)), 'tuple(c.shape) == ((M, N // 2) if swiglu else (M, N))')
    _require(not (swiglu and accumulate), 'not (swiglu and accumulate)')
    _same_dtype(a, b)
    epi = BIV_EPI_SWIGLU if swiglu else (BIV_EPI_ACCUM if accumulate else BIV_EPI_STORE)
    _check("gemm_bi", _lib.gemm_bi(_p(a), _p(b), _p(c), M, N, K, _dt(a), _dt(c), epi, _stream()))
    return c


SWIGLU_BLOCK = 32


def pack_gate_up(w_gate_up):
    """[W_gate; W_up] ([2F, H]) -> the BIV_EPI_SWIGLU layout: blocks of 32 gate
    rows followed by the 32 matching up rows (a copy; layout only)."""
    F2, H = w_gate_up.shape
    F = F2 // 2
    _require(F2 == 2 * F and F % SWIGLU_BLOCK == 0, 'F2 == 2 * F and F % SWIGLU_BLOCK == 0')
    return w_gate_up.view(2, F // SWIGLU_BLOCK, SWIGLU_BLOCK, H).transpose(0, 1).contiguous().view(F2, H)


def attn_workspace_bytes(R, Hkv, max_blocks, seg_tokens=ATTN_SEG_TOKENS, q_len=1, Hq=None):
    """Workspace of the bf16 attention for R requests of q_len rows (Hq query
    heads; needed once q_len * Hq/Hkv > 32, i.e. several row blocks)."""
    if Hq is None:
        return _lib.biv_attn_workspace_bytes(R, Hkv, max_blocks, seg_tokens)
    return _lib.biv_attn_workspace_bytes_q(R, q_len, Hq, Hkv, max_blocks, seg_tokens)


def _attn_checks(q, k_cache, v_cache, block_table, ctx, out, q_len, q_off=None):
    """q: [T, Hq*D] row view (row stride may exceed Hq*D) or [T, Hq, D]; out [T, Hq, D] contiguous.
    T = R*q_len, or with q_off (device int32 [R+1]) the caller's q_off[R]."""
    if q.stride(-1) != 1:
        raise ValueError("q rows must be contiguous")
    _same_dtype(q, k_cache, v_cache, out)
    _want(block_table, torch.int32, "block_table")
    _want(ctx, torch.int32, "ctx")
    T, Hq, D = out.shape
    if q.dim() == 3:
        _require(q.stride(1) == D and tuple(q.shape) == (T, Hq, D), 'q.stride(1) == D and tuple(q.shape) == (T, Hq, D)')
    else:
        _require(tuple(q.shape) == (T, Hq * D), 'tuple(q.shape) == (T, Hq * D)')
    R, _ = block_table.shape
    _require(ctx.numel() == R, "ctx [R]")
    if q_off is None:
        _require(T == R * q_len, "rows = R * q_len")
    else:
        _want(q_off, torch.int32, "q_off")
        _require(q_off.numel() == R + 1 and q_off.is_cuda, "q_off: device int32 [R+1]")
        _require(T <= R * q_len, "rows <= R * q_len (q_len: the most rows of any request)")
    _require(k_cache.shape == v_cache.shape and k_cache.dim() == 4 and k_cache.shape[2] == 16 and k_cache.shape[3] == D, 'k_cache.shape == v_cache.shape and k_cache.dim() == 4 and k_cache.shape[2] == 16 and k_cache.shape[3] == D')
    return q.stride(0), Hq, D


def attn_decode_bi(q, k_cache, v_cache, block_table, ctx, out, q_len, scale, workspace=None, q_off=None):
    """q [T, Hq*D] (rows may be strided) or [T, Hq, D]; out [T, Hq, D];
    caches [num_blocks, Hkv, 16, D]; block_table [R, max_blocks] int32; ctx [R] int32.
    Without q_off every request has q_len rows (T = R*q_len); with q_off (device
    int32 [R+1], q_off[R] = T) request r has rows q_off[r] .. q_off[r+1]-1 and
    q_len is the most rows of any request."""
    _contig(k_cache, v_cache, block_table, ctx, out, q_off)
    q_stride, Hq, D = _attn_checks(q, k_cache, v_cache, block_table, ctx, out, q_len, q_off)
    R, max_blocks = block_table.shape
    num_blocks, Hkv = k_cache.shape[0], k_cache.shape[1]
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("attn_decode_bi", _lib.attn_decode_bi(
        _p(q), q_stride, _p(k_cache), _p(v_cache), _p(block_table), _p(ctx), _p(q_off), _p(out), R, q_len, Hq, Hkv, D,
        max_blocks, num_blocks, scale, _dt(q), _p(workspace), wbytes, _stream()))
    return out


ATTN_STATIC_SCRATCH_BYTES = 32 << 20


def attn_decode_bi_static(q, k_cache, v_cache, block_table, ctx, out, q_len, scale, q_off=None):
    """attn_decode_bi with its workspace in the library's static per-GPU
    scratch (allocates nothing; for callers that cannot allocate).  Calls
    whose workspace would exceed ATTN_STATIC_SCRATCH_BYTES raise; calls that
    overlap on one GPU race (order them on one stream)."""
    _contig(k_cache, v_cache, block_table, ctx, out, q_off)
    q_stride, Hq, D = _attn_checks(q, k_cache, v_cache, block_table, ctx, out, q_len, q_off)
    R, max_blocks = block_table.shape
    num_blocks, Hkv = k_cache.shape[0], k_cache.shape[1]
    _check("attn_decode_bi_static", _lib.attn_decode_bi_static(
        _p(q), q_stride, _p(k_cache), _p(v_cache), _p(block_table), _p(ctx), _p(q_off), _p(out), R, q_len, Hq, Hkv, D,
        max_blocks, num_blocks, scale, _dt(q), _stream()))
    return out


def attn_adaptive_split(R, Hkv, max_blocks):
    return _lib.biv_attn_adaptive_split(R, Hkv, max_blocks)


def attn_decode_adaptive(q, k_cache, v_cache, block_table, ctx, out, q_len, scale, workspace, split_tokens=0):
    _contig(k_cache, v_cache, block_table, ctx, out)
    q_stride, Hq, D = _attn_checks(q, k_cache, v_cache, block_table, ctx, out, q_len)
    R, max_blocks = block_table.shape
    num_blocks, Hkv = k_cache.shape[0], k_cache.shape[1]
    wbytes = workspace.numel() * workspace.element_size()
    _check("attn_decode_adaptive", _lib.attn_decode_adaptive(
        _p(q), q_stride, _p(k_cache), _p(v_cache), _p(block_table), _p(ctx), _p(out), R, q_len, Hq, Hkv, D, max_blocks,
        num_blocks, scale, split_tokens, _p(workspace), wbytes, _stream()))
    return out


def kv_copy_pages(src_page, dst_page, k_cache, v_cache):
    """Whole-page copies inside one layer's cache: page dst_page[i] <- src_page[i]
    (int32 [n] device tensors); caches [num_blocks, Hkv, 16, D]."""
    _contig(src_page, dst_page, k_cache, v_cache)
    _want(src_page, torch.int32, "src_page")
    _want(dst_page, torch.int32, "dst_page")
    _require(src_page.numel() == dst_page.numel(), 'src_page.numel() == dst_page.numel()')
    _same_dtype(k_cache, v_cache)
    nb, Hkv, blk, D = k_cache.shape
    _require(blk == 16 and tuple(v_cache.shape) == tuple(k_cache.shape), 'blk == 16 and tuple(v_cache.shape) == tuple(k_cache.shape)')
    _check("kv_copy_pages", _lib.kv_copy_pages(_p(src_page), _p(dst_page), src_page.numel(), _p(k_cache), _p(v_cache),
                                               nb, Hkv, D, _dt(k_cache), _stream()))


def tree_select(accept_len, next_token, best, accept_out, next_out):
    """accept_len/next_token [R, B] int32 (B chains per request); best, accept_out,
    next_out [R] int32: the chain with the longest accepted prefix (lowest index
    among equals) and its values."""
    _contig(accept_len, next_token, best, accept_out, next_out)
    for t, n in ((accept_len, "accept_len"), (next_token, "next_token"), (best, "best"),
                 (accept_out, "accept_out"), (next_out, "next_out")):
        _want(t, torch.int32, n)
    R, B = accept_len.shape
    _require(tuple(next_token.shape) == (R, B) and best.numel() == R and accept_out.numel() == R and next_out.numel() == R, 'tuple(next_token.shape) == (R, B) and best.numel() == R and accept_out.numel() == R and next_out.numel() == R')
    _check("tree_select", _lib.tree_select(_p(accept_len), _p(next_token), R, B, _p(best), _p(accept_out),
                                           _p(next_out), _stream()))


def gumbel_verify(logits, noise, cand, target, accept_len, next_token):
    """logits/noise [R*K, V] fp32; cand/target [R, K] int32; accept_len/next_token [R] int32."""
    _contig(logits, noise, cand, target, accept_len, next_token)
    _want(logits, torch.float32, "logits")
    _want(noise, torch.float32, "noise")
    for t, n in ((cand, "cand"), (target, "target"), (accept_len, "accept_len"), (next_token, "next_token")):
        _want(t, torch.int32, n)
    R, K = cand.shape
    V = logits.shape[-1]
    _require(logits.numel() == R * K * V and noise.numel() == R * K * V, 'logits.numel() == R * K * V and noise.numel() == R * K * V')
    _require(target.numel() == R * K and accept_len.numel() == R and next_token.numel() == R, 'target.numel() == R * K and accept_len.numel() == R and next_token.numel() == R')
    _check("gumbel_verify", _lib.gumbel_verify(_p(logits), _p(noise), _p(cand), R, K, V, _p(target),
                                               _p(accept_len), _p(next_token), _stream()))
    return target, accept_len, next_token


def gumbel_topk(logits, noise, idx, score=None):
    """idx [rows, k] int32 (and score [rows, k] fp32) <- the k largest
    fl32(logit + noise) of each row of logits/noise [rows, V] fp32."""
    _contig(logits, noise, idx)
    _want(logits, torch.float32, "logits")
    _want(noise, torch.float32, "noise")
    _want(idx, torch.int32, "idx")
    rows, k = idx.shape
    V = logits.shape[-1]
    _require(logits.numel() == rows * V and noise.numel() == rows * V, 'logits.numel() == rows * V and noise.numel() == rows * V')
    if score is not None:
        _contig(score)
        _want(score, torch.float32, "score")
        _require(tuple(score.shape) == (rows, k), 'tuple(score.shape) == (rows, k)')
    _check("gumbel_topk", _lib.gumbel_topk(_p(logits), _p(noise), rows, V, k, _p(idx),
                                           _p(score) if score is not None else None, _stream()))


def gumbel_workspace_bytes(M, V):
    """Workspace bytes of lm_head_gumbel_verify for M = R*K rows and vocabulary V."""
    return _lib.biv_gumbel_workspace_bytes(M, V)


def lm_head_gumbel_verify(h, w_head, noise, cand, target, accept_len, next_token, workspace):
    """lm_head matmul + Gumbel verification without fp32 logits in memory.
    h [R*K, H] bf16, w_head [V, H] bf16, noise [R*K, V] fp32, cand/target
    [R, K] int32, accept_len/next_token [R] int32; same results as gemm_bi to
    fp32 logits followed by gumbel_verify."""
    _contig(h, w_head, noise, cand, target, accept_len, next_token, workspace)
    _want(h, torch.bfloat16, "h")
    _want(w_head, torch.bfloat16, "w_head")
    _want(noise, torch.float32, "noise")
    for t, n in ((cand, "cand"), (target, "target"), (accept_len, "accept_len"), (next_token, "next_token")):
        _want(t, torch.int32, n)
    R, K = cand.shape
    V, H = w_head.shape
    _require(tuple(h.shape) == (R * K, H) and noise.numel() == R * K * V, 'tuple(h.shape) == (R * K, H) and noise.numel() == R * K * V')
    _require(target.numel() == R * K and accept_len.numel() == R and next_token.numel() == R, 'target.numel() == R * K and accept_len.numel() == R and next_token.numel() == R')
    _check("lm_head_gumbel_verify", _lib.lm_head_gumbel_verify(
        _p(h), _p(w_head), _p(noise), _p(cand), R, K, V, H, _p(target), _p(accept_len), _p(next_token),
        _p(workspace), workspace.numel() * workspace.element_size(), _stream()))


def kv_overwrite(k_new, v_new, slot, k_cache, v_cache):
    """k_new/v_new: [T, Hkv*D] views (row stride may exceed Hkv*D); slot [T] int64."""
    T = slot.shape[0]
    num_blocks, Hkv, _, D = k_cache.shape
    _same_dtype(k_new, v_new, k_cache, v_cache)
    _want(slot, torch.int64, "slot")
    stride = k_new.stride(0)
    _require(v_new.stride(0) == stride and k_new.stride(-1) == 1 and v_new.stride(-1) == 1, 'v_new.stride(0) == stride and k_new.stride(-1) == 1 and v_new.stride(-1) == 1')
    _require(tuple(k_new.shape) == (T, Hkv * D) and tuple(v_new.shape) == (T, Hkv * D), 'tuple(k_new.shape) == (T, Hkv * D) and tuple(v_new.shape) == (T, Hkv * D)')
    _require(k_cache.shape == v_cache.shape, 'k_cache.shape == v_cache.shape')
    _contig(slot, k_cache, v_cache)
    _check("kv_overwrite", _lib.kv_overwrite(_p(k_new), _p(v_new), stride, _p(slot), _p(k_cache), _p(v_cache),
                                             T, Hkv, D, num_blocks, _dt(k_cache), _stream()))


def embed_rows(ids, table, out):
    _contig(ids, table, out)
    _want(ids, torch.int32, "ids")
    V, H = table.shape
    _require(tuple(out.shape) == (ids.shape[0], H), 'tuple(out.shape) == (ids.shape[0], H)')
    _check("embed_rows", _lib.embed_rows(_p(ids), _p(table), _dt(table), _p(out), _dt(out), ids.shape[0], V, H,
                                         _stream()))
    return out


def rope_table(max_pos, D, theta):
    """Host fp32 table [max_pos, D/2, 2] (cos, sin) made by the library."""
    t = torch.empty((max_pos, D // 2, 2), dtype=torch.float32)
    _check("biv_rope_table", _lib.biv_rope_table(ctypes.c_void_p(t.data_ptr()), max_pos, D, theta))
    return t


def rope_apply(x, pos, cos_sin, n_heads, D):
    """In place on the first n_heads*D columns of each row of x (row stride x.stride(0))."""
    _require(x.stride(-1) == 1 and x.shape[1] >= n_heads * D, 'x.stride(-1) == 1 and x.shape[1] >= n_heads * D')
    _contig(pos, cos_sin)
    _want(pos, torch.int32, "pos")
    _want(cos_sin, torch.float32, "cos_sin")
    _require(pos.numel() == x.shape[0] and cos_sin.shape[1] * 2 == D, 'pos.numel() == x.shape[0] and cos_sin.shape[1] * 2 == D')
    _check("rope_apply", _lib.rope_apply(_p(x), x.stride(0), _p(pos), _p(cos_sin), x.shape[0], n_heads, D,
                                         cos_sin.shape[0], _dt(x), _stream()))


def rope_kv_overwrite(qkv, pos, cos_sin, slot, k_cache, v_cache, n_q_heads):
    """rope_apply on the Q and K heads of the fused QKV rows, then kv_overwrite
    of their K and V heads, in one pass (same bits as the two calls)."""
    T = qkv.shape[0]
    num_blocks, Hkv, _, D = k_cache.shape
    _require(qkv.stride(-1) == 1 and qkv.shape[1] >= (n_q_heads + 2 * Hkv) * D, 'qkv.stride(-1) == 1 and qkv.shape[1] >= (n_q_heads + 2 * Hkv) * D')
    _same_dtype(qkv, k_cache, v_cache)
    _contig(pos, cos_sin, slot, k_cache, v_cache)
    _want(pos, torch.int32, "pos")
    _want(cos_sin, torch.float32, "cos_sin")
    _want(slot, torch.int64, "slot")
    _require(pos.numel() == T and slot.numel() == T and cos_sin.shape[1] * 2 == D, 'pos.numel() == T and slot.numel() == T and cos_sin.shape[1] * 2 == D')
    _require(k_cache.shape == v_cache.shape, 'k_cache.shape == v_cache.shape')
    _check("rope_kv_overwrite", _lib.rope_kv_overwrite(_p(qkv), qkv.stride(0), _p(pos), _p(cos_sin), _p(slot),
                                                       _p(k_cache), _p(v_cache), T, n_q_heads, Hkv, D,
                                                       cos_sin.shape[0], num_blocks, _dt(qkv), _stream()))


def swiglu(gu, out, block=0):
    """out = silu(gate) * up; gate/up are the row halves of gu (block 0) or its
    interleaved blocks (block = SWIGLU_BLOCK for the packed gate/up weight)."""
    _contig(gu, out)
    _same_dtype(gu, out)
    M, N2 = gu.shape
    _require(tuple(out.shape) == (M, N2 // 2), 'tuple(out.shape) == (M, N2 // 2)')
    _check("swiglu", _lib.swiglu(_p(gu), _p(out), M, N2 // 2, block, _dt(gu), _stream()))
    return out


def splitk_workspace_bytes(M, N, splits):
    return _lib.biv_splitk_workspace_bytes(M, N, splits)


def splitk_auto_splits(M, N, K):
    return _lib.biv_splitk_auto_splits(M, N, K)


def gemm_splitk(a, b, c, splits, workspace, accumulate=False, swiglu=False):
    """Split-K comparison matmul (not batch invariant); epilogues as gemm_bi's."""
    _contig(a, b, c, workspace)
    _want(a, torch.bfloat16, "a")
    _want(b, torch.bfloat16, "b")
    M, K = a.shape
    N = b.shape[0]
    _require(b.shape[1] == K and tuple(c.shape) == ((M, N // 2) if swiglu else (M, N)), "gemm_splitk shapes")
    _require(not (swiglu and accumulate), "swiglu and accumulate together")
    epi = BIV_EPI_SWIGLU if swiglu else (BIV_EPI_ACCUM if accumulate else BIV_EPI_STORE)
    _check("gemm_splitk", _lib.gemm_splitk(_p(a), _p(b), _p(c), M, N, K, _dt(c), epi, splits, _p(workspace),
                                           workspace.numel() * workspace.element_size(), _stream()))
    return c


def abi_version():
    return _lib.biv_abi_version()
