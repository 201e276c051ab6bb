"""Deterministic prefill with the batch-invariant kernels, on the
Llama-3-8B-shaped slice (2 of the 32 layers, bf16).

A prompt of P tokens runs as one forward of P rows (q_len = P from context 0:
the attention takes the rows in 32-row blocks, each with the keys up to its
own last row).  LLM-42 post, paragraphs 1 and 3: with batch-invariant kernels
a token's numbers do not depend on how many others are computed with it, so
the prompt's K/V and every row's logits must be bit for bit those of feeding
the prompt one token at a time.  That is what lets the verifier start from a
prompt cache that decoding itself would have produced.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from gpu_util import DEV, announce, bits, sync

pytestmark = pytest.mark.gpu

LAYERS, P = 2, 300


def test_prefill_equals_token_by_token_decode():
    import invariant_verify_verifier_amd.verifier as V

    assert torch.cuda.is_available()
    sh = wl.LLAMA3_8B
    dw = wl.device_model_weights(sh, 60, layers=LAYERS)
    shape = V.Shape(LAYERS, sh.hidden, sh.heads, sh.kv_heads, sh.head_dim, sh.ffn, sh.vocab, sh.eps, sh.rope_theta)
    model = V.VerifierModel(shape, torch.bfloat16, dw["layers"], dw["embed"], dw["lm_head"], dw["final_norm"],
                            max_pos=4096)
    lay = wl.paged_layout(np.array([0], np.int32), P, seed=61, spare_blocks=4)
    bt = torch.from_numpy(lay.block_table).to(DEV)
    pos = np.arange(P, dtype=np.int32)
    slots = (lay.block_table[0, pos // 16].astype(np.int64) * 16 + pos % 16)
    toks = wl.tokens(62, (P,), sh.vocab)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    cache_a = model.alloc_kv(lay.num_blocks)
    cache_b = model.alloc_kv(lay.num_blocks)
    announce("prefill", P, "tokens in one forward")
    logits_p = model.forward(dev(toks), dev(pos), dev(np.array([0], np.int32)), P, bt, dev(slots), cache_a).clone()
    sync()
    announce("prefill: the same prompt one token at a time")
    step_bits = []
    for j in range(P):
        lg = model.forward(dev(toks[j:j + 1]), dev(pos[j:j + 1]), dev(np.array([j], np.int32)), 1, bt,
                           dev(slots[j:j + 1]), cache_b)
        step_bits.append(bits(lg)[0].copy())
    sync()
    full = bits(logits_p)
    for j in range(P):
        assert np.array_equal(step_bits[j], full[j]), f"logits of prompt row {j}"
    used = np.unique(lay.block_table[0, :(P + 15) // 16])
    for li, ((ka, va), (kb, vb)) in enumerate(zip(cache_a, cache_b)):
        idx = torch.from_numpy(used).to(DEV)
        assert torch.equal(ka[idx].view(torch.int16), kb[idx].view(torch.int16)), f"K cache layer {li}"
        assert torch.equal(va[idx].view(torch.int16), vb[idx].view(torch.int16)), f"V cache layer {li}"
