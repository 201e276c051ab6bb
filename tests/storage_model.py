"""Precision model of the bf16 verifier step, from which its end-to-end
logit bound is derived (test infrastructure; built only from the oracle's own plain
operations).

The bf16 step computes every matmul, norm and attention with fp32 (or wider)
arithmetic, but stores activations between its kernels as bf16 and its
residual stream as fp32.  Those stores are where almost all of its error
against the fp64 oracle comes from.  ``bf16_storage_forward`` is the oracle's
decoder forward (LLM-42 post, paragraphs 3-4: the verifier forward over the
K candidates of each request, its K/V written before attention) with exactly
those stores inserted -- each a single rounding of the fp64 value -- and
fp64 arithmetic everywhere else:

  h   = bf16(rmsnorm(x))              before the QKV and gate/up matmuls
  qkv = bf16(h Wqkv^T)                the QKV matmul's output
  q,k = bf16(rope(q)), bf16(rope(k))  RoPE in place on the bf16 rows
  a   = bf16(attention(q, cache))     the attention output
  x   = fp32(x + a Wo^T)              the residual add in the O matmul
  act = bf16(silu(g) * u)             SwiGLU on the unrounded gate/up results
  x   = fp32(x + act Wd^T)            the residual add in the down matmul
  logits = fp32(bf16(rmsnorm(x)) W_lm^T)

Its difference from the fp64 oracle is what bf16 storage costs, computed
without the GPU.  The step rounds at the same points, but its values before
each rounding differ slightly from the model's (fp32 accumulation order, fp32
transcendentals, the RoPE table's fp32 angles, the bf16 attention
probabilities of its PV product).  Where such a difference straddles a bf16
rounding boundary the two round to neighbouring values, and that difference
is carried into every later rounding, where it straddles boundaries far more
often: a few layers in, the step's roundings are independent draws from the
same distribution as the model's.  The step's logit error is therefore a
second sample of the model's error distribution, not a copy of it (measured
on the 2-layer slice: |step - model| 0.054 against |model - fp64| 0.053).

The bound used by the parity tests is statistical and fixed in its ratios:
  * RMS over the checked logits of (step - fp64) <= RMS_RATIO * the model's;
  * max |step - fp64| <= MAX_RATIO * the model's max.
A row's logit errors are W_lm times the error of that row's final hidden
vector, so their RMS over the vocabulary is set by the norm of a 4096-element
error vector built from many independent roundings: two samples agree to a
few percent.  Their maxima (~5 standard deviations out over ~10^5 logits
per row) agree to ~10%.  RMS_RATIO = 1.15 and MAX_RATIO = 1.5 leave room for
that and for the step's few extra fp32 effects, while a step whose typical
error grew by a fifth would fail.
"""
import numpy as np

import oracle

RMS_RATIO = 1.15
MAX_RATIO = 1.5


def error_bound(model_logits, fp64_logits):
    """(rms bound, max bound) for the step's logits against the fp64 ones."""
    d = np.asarray(model_logits, dtype=np.float64) - np.asarray(fp64_logits, dtype=np.float64)
    return RMS_RATIO * float(np.sqrt(np.mean(d * d))), MAX_RATIO * float(np.abs(d).max())


def _bf16(a):
    return oracle.round_bf16(a)


def _fp32(a):
    return np.asarray(a, dtype=np.float64).astype(np.float32).astype(np.float64)


def bf16_storage_forward(w, tokens, ctx, k_caches, v_caches, block_table, block=16):
    """The oracle's decoder forward with the bf16 step's stores (see the
    module docstring).  Arguments as for oracle.decoder_forward; the caches
    (fp64 copies holding bf16 values) are modified in place.  Returns fp32
    logits as fp64 [R*q_len, V]."""
    sh = w["shape"]
    tokens = np.asarray(tokens)
    R, q_len = tokens.shape
    W = R * q_len
    Hq, Hkv, D = sh.heads, sh.kv_heads, sh.head_dim
    pos = (np.asarray(ctx, dtype=np.int64)[:, None] + np.arange(q_len)[None, :]).reshape(-1)
    slots = np.array([int(block_table[t // q_len][int(p) // block]) * block + int(p) % block
                      for t, p in enumerate(pos)], dtype=np.int64)
    x = _fp32(w["embed"][tokens.reshape(-1)])
    scale = 1.0 / np.sqrt(D)
    qc, kc = Hq * D, Hkv * D
    for li, L in enumerate(w["layers"]):
        h = _bf16(oracle.rmsnorm(x, L["attn_norm"], sh.eps))
        wqkv = np.concatenate([L["wq"], L["wk"], L["wv"]], axis=0)
        qkv = _bf16(oracle.linear(h, wqkv))
        q = _bf16(oracle.rope(qkv[:, :qc].reshape(W, Hq, D), pos, sh.rope_theta))
        k = _bf16(oracle.rope(qkv[:, qc:qc + kc].reshape(W, Hkv, D), pos, sh.rope_theta))
        v = qkv[:, qc + kc:].reshape(W, Hkv, D)
        oracle.kv_overwrite(k_caches[li], v_caches[li], k, v, slots, block)
        a = _bf16(oracle.attention(q, k_caches[li], v_caches[li], block_table, ctx, q_len, scale, block))
        x = _fp32(x + oracle.linear(a.reshape(W, qc), L["wo"]))
        h = _bf16(oracle.rmsnorm(x, L["ffn_norm"], sh.eps))
        act = _bf16(oracle.silu(oracle.linear(h, L["w_gate"])) * oracle.linear(h, L["w_up"]))
        x = _fp32(x + oracle.linear(act, L["w_down"]))
    return _fp32(oracle.linear(_bf16(oracle.rmsnorm(x, w["final_norm"], sh.eps)), w["lm_head"]))
