"""attn_decode_bi_static, the allocation-free attention entry point (its
workspace is the library's static per-GPU scratch), against attn_decode_bi
with a caller workspace: the same kernels, so the same bits, on two calls in a
row -- the second smaller, reusing the scratch the first left behind -- and a
call whose workspace would not fit is refused before any launch."""
import math

import numpy as np
import pytest
import torch

import workloads as wl
from gpu_util import DEV, announce, bits, dev_bf16, dev_i32, sync

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def biv():
    import invariant_verify_verifier_amd as m

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def _case(biv, ctx, q_len, seed, q_off=None):
    Hq, Hkv, D = 32, 8, 128
    R = len(ctx)
    lay = wl.paged_layout(ctx, q_len, seed=seed, spare_blocks=3)
    kc = dev_bf16(wl.normal_bf16(seed + 1, (lay.num_blocks, Hkv, 16, D)))
    vc = dev_bf16(wl.normal_bf16(seed + 2, (lay.num_blocks, Hkv, 16, D)))
    T = R * q_len if q_off is None else int(q_off[-1])
    q = dev_bf16(wl.normal_bf16(seed + 3, (T, Hq, D)))
    bt, cx = dev_i32(lay.block_table), dev_i32(lay.ctx)
    qo = None if q_off is None else dev_i32(q_off)
    ws = torch.zeros(biv.attn_workspace_bytes(R, Hkv, lay.max_blocks, q_len=q_len, Hq=Hq), dtype=torch.uint8,
                     device=DEV)
    ref = torch.full((T, Hq, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    got = torch.full((T, Hq, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    scale = 1.0 / math.sqrt(D)
    announce("attn_decode_bi_static", R, q_len, seed)
    biv.attn_decode_bi(q, kc, vc, bt, cx, ref, q_len, scale, ws, q_off=qo)
    biv.attn_decode_bi_static(q, kc, vc, bt, cx, got, q_len, scale, q_off=qo)
    sync()
    return bits(ref), bits(got)


def test_static_scratch_attention_equals_workspace_call(biv):
    # first call: 64 requests of up to two 4096-token segments, K = 8 rows
    # (segment partials: ~17 MB of the scratch)
    ctx = list(wl.rng(200).integers(500, 8000, size=64))
    ref, got = _case(biv, ctx, 8, seed=201)
    assert np.array_equal(got, ref)
    # second, smaller call (one request, one row: its segments split over 16
    # waves, chunk partials in the scratch) over what the first left there
    ref, got = _case(biv, [9000], 1, seed=210)
    assert np.array_equal(got, ref)
    # ragged rows through the same scratch
    off = np.array([0, 3, 11, 12], np.int32)
    ref, got = _case(biv, [300, 5000, 70], 8, seed=220, q_off=off)
    assert np.array_equal(got, ref)


def test_static_scratch_refuses_oversized_calls(biv):
    """A workspace beyond the static scratch is refused with an error before
    anything launches (nothing is allocated instead)."""
    Hq, Hkv, D = 32, 8, 128
    R, max_blocks = 64, 2048  # contexts up to 32768: 64 x 8 x 8 segment partials > 32 MiB
    assert biv.attn_workspace_bytes(R, Hkv, max_blocks) > biv.ATTN_STATIC_SCRATCH_BYTES
    kc = torch.zeros((4, Hkv, 16, D), dtype=torch.bfloat16, device=DEV)
    q = torch.zeros((R, Hq, D), dtype=torch.bfloat16, device=DEV)
    out = torch.zeros_like(q)
    bt = torch.zeros((R, max_blocks), dtype=torch.int32, device=DEV)
    cx = torch.zeros(R, dtype=torch.int32, device=DEV)
    with pytest.raises(biv.BivError, match="static scratch"):
        biv.attn_decode_bi_static(q, kc, kc, bt, cx, out, 1, 0.1)
