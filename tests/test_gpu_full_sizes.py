"""Attention at the full size of the batch-invariant decode-attention workload
(LLM-42 post, paragraph 1: fixed KV-split size; paragraphs 3-4: the verifier's
K rows per request): 256 requests with contexts U[512, 32768], 32 Q / 8 KV
heads x 128, 16-token pages placed by a seeded permutation, K/V ~ N(0, 1)
bf16, in the launch configuration the benchmark times.

The oracle cannot take all 256 requests (about 17 GB of cache), so it checks
sampled requests one by one -- the longest, the shortest and a seeded random
handful -- on host copies of their own pages; two of them are also run alone
and must give the same bits as inside the full batch.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_util import DEV, announce, bits, dev_i32, f64, sync
from tolerances import check_bf16

pytestmark = pytest.mark.gpu

R, HQ, HKV, D = 256, 32, 8, 128


@pytest.fixture(scope="module")
def biv():
    import invariant_verify_verifier_amd as m

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


@pytest.fixture(scope="module")
def cache():
    ctx = wl.context_lengths(wl.SEEDS["attn_len"], R, 512, 32768)
    lay = wl.paged_layout(ctx, 8, seed=wl.SEEDS["attn_perm"])
    announce("full-size attention cache", lay.num_blocks, "blocks")
    kc = wl._torch_normal((lay.num_blocks, HKV, 16, D), wl.SEEDS["attn_qkv"], 1, 1.0, DEV, torch.bfloat16)
    vc = wl._torch_normal((lay.num_blocks, HKV, 16, D), wl.SEEDS["attn_qkv"], 2, 1.0, DEV, torch.bfloat16)
    yield lay, kc, vc
    del kc, vc
    torch.cuda.empty_cache()


def _run(biv, q, kc, vc, bt, cx, q_len):
    Rr = bt.shape[0]
    out = torch.full((Rr * q_len, HQ, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    ws = torch.zeros(biv.attn_workspace_bytes(Rr, HKV, bt.shape[1]), dtype=torch.uint8, device=DEV)
    biv.attn_decode_bi(q, kc, vc, bt, cx, out, q_len, 1.0 / math.sqrt(D), ws)
    sync()
    return out


def _oracle_rows(lay, kc, vc, q_host, r, q_len):
    """The oracle on request r alone, from host copies of its pages."""
    pages = [int(p) for p in lay.block_table[r] if p >= 0]
    idx = torch.tensor(pages, device=DEV)
    k64, v64 = f64(kc[idx]), f64(vc[idx])
    bt = np.full((1, lay.max_blocks), -1, np.int32)
    bt[0, :len(pages)] = np.arange(len(pages))
    return oracle.attention(q_host[r * q_len:(r + 1) * q_len], k64, v64, bt, lay.ctx[r:r + 1], q_len,
                            1.0 / math.sqrt(D))


@pytest.mark.parametrize("q_len", [1, 8])
def test_attention_full_size_sampled_parity_and_invariance(biv, cache, q_len):
    lay, kc, vc = cache
    q = wl._torch_normal((R * q_len, HQ, D), wl.SEEDS["attn_qkv"], 10 + q_len, 1.0, DEV, torch.bfloat16)
    bt, cx = dev_i32(lay.block_table), dev_i32(lay.ctx)
    announce("full-size attention B=256 q_len", q_len)
    out = _run(biv, q, kc, vc, bt, cx, q_len)
    got = f64(out)
    assert np.isfinite(got).all()
    q_host = f64(q)
    pick = {int(np.argmax(lay.ctx)), int(np.argmin(lay.ctx))}
    pick |= {int(x) for x in wl.rng(70 + q_len).choice(R, size=4, replace=False)}
    for r in sorted(pick):
        announce("full-size attention oracle request", r, "ctx", int(lay.ctx[r]))
        ref = _oracle_rows(lay, kc, vc, q_host, r, q_len)
        check_bf16(got[r * q_len:(r + 1) * q_len], ref, f"request {r} (ctx {lay.ctx[r]}) q_len={q_len}")
    # the same request alone (its own one-row block table): identical bits
    full_bits = bits(out)
    for r in sorted(pick)[:2]:
        announce("full-size attention alone request", r)
        alone = _run(biv, q[r * q_len:(r + 1) * q_len].contiguous(), kc, vc, bt[r:r + 1].contiguous(),
                     cx[r:r + 1].contiguous(), q_len)
        assert np.array_equal(bits(alone), full_bits[r * q_len:(r + 1) * q_len]), f"request {r} changed alone"
