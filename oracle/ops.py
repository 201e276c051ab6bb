"""Plain fp64 definitions of the verifier step (oracle; test infrastructure only).

Citations name the page and the paragraph a function follows:

* "LLM-42 post" = the Telegram post on batch-invariant kernels and LLM-42's
  decode-verify-rollback (paragraph 1: batch-invariant matmul/RMSNorm/attention;
  paragraph 3: fast path, verifier, overwrite of fast-path KV; paragraph 4:
  W = N*K).
* "Gumbel post" = the reading-club post on "Coupling without Communication and
  Drafter-Invariant Speculative Decoding" (Gumbel-max trick; Gumbel coupling;
  token comparison; drafter invariance).
* "spec-dec guide" = the news piece on NVIDIA's speculative-decoding guide
  (speculative decoding is lossless: the target accepts only tokens it would
  write itself).

Where the pages are silent (RoPE convention, layer order, norm epsilon, what
happens when all K candidates are accepted, ...) the plainest reading is
taken, and the function or section that takes it says which (the RoPE
section header, the decoder's pre-norm layer order, verify's rule for an
all-accepted request).
"""
from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# Input decoding (bits in, fp64 out) and bf16 rounding of a reference
# ---------------------------------------------------------------------------


def as_f64(a, dtype: str) -> np.ndarray:
    """Inputs as fp64.  ``dtype`` "bf16": uint16 bit patterns; "f32": fp32."""
    a = np.asarray(a)
    if dtype == "bf16":
        return (a.astype(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if dtype == "f32":
        return a.astype(np.float32).astype(np.float64)
    raise ValueError(dtype)


def round_bf16(x) -> np.ndarray:
    """fp64 -> nearest bf16 value (ties to even), rounded ONCE, returned as fp64.

    Used to state bf16-output tolerances against the exact value.  Works on
    the fp64 significand directly (no detour through fp32, which could round
    twice).  Normal range only; bf16 subnormals are flushed like fp32 ones are
    not needed by any workload here.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)  # x = m * 2^e, 0.5 <= |m| < 1
    q = np.rint(m * 256.0)  # 8 significant bits, rint = ties-to-even
    return np.ldexp(q / 256.0, e)


# ---------------------------------------------------------------------------
# O1 RMSNorm — LLM-42 post, paragraph 1 (RMSNorm with a fixed split over hidden)
# ---------------------------------------------------------------------------


def rmsnorm(x, gamma, eps) -> np.ndarray:
    """y = x * gamma / sqrt(mean(x^2) + eps), mean over the last (hidden) axis."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(gamma, dtype=np.float64)


# ---------------------------------------------------------------------------
# O2 matmul — LLM-42 post, paragraph 1 (data-parallel tiling, no split-K)
# ---------------------------------------------------------------------------


def linear(a, w) -> np.ndarray:
    """out[m, n] = sum_k a[m, k] * w[n, k]   (w in [out_features, in_features])."""
    return np.asarray(a, dtype=np.float64) @ np.asarray(w, dtype=np.float64).T


def silu(z) -> np.ndarray:
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


# ---------------------------------------------------------------------------
# O3 RoPE (not on the pages: rotate-half convention, theta = 500000)
# ---------------------------------------------------------------------------


def rope(x, positions, theta) -> np.ndarray:
    """x [T, heads, D]; pair (i, i + D/2) rotated by angle pos * theta^(-2i/D)."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    half = D // 2
    inv = theta ** (-2.0 * np.arange(half, dtype=np.float64) / D)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv[None, :]  # [T, half]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


# ---------------------------------------------------------------------------
# O4 attention — LLM-42 post, paragraph 1 (attention with a fixed KV split)
# ---------------------------------------------------------------------------


def _gather_positions(cache, block_table_row, n, block):
    """cache [num_blocks, Hkv, block, D] -> [n, Hkv, D] for positions 0..n-1."""
    p = np.arange(n)
    pages = np.asarray(block_table_row)[p // block]
    return cache[pages, :, p % block, :]


def attention(q, k_cache, v_cache, block_table, ctx, q_len, scale, block=16) -> np.ndarray:
    """Paged causal decode/verify attention with grouped KV heads.

    q [R*q_len, Hq, D]; caches [num_blocks, Hkv, block, D]; row (r, j) is the
    query at absolute position ctx[r] + j and attends to keys 0..ctx[r]+j;
    q head h reads KV head h // (Hq/Hkv).  Plain full softmax in fp64.
    """
    q = np.asarray(q, dtype=np.float64)
    R = len(ctx)
    Hq, D = q.shape[1], q.shape[2]
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    out = np.zeros_like(q)
    for r in range(R):
        n_all = int(ctx[r]) + q_len
        K = _gather_positions(k_cache, block_table[r], n_all, block).astype(np.float64)
        V = _gather_positions(v_cache, block_table[r], n_all, block).astype(np.float64)
        for j in range(q_len):
            n = int(ctx[r]) + j + 1
            for h in range(Hq):
                kh = h // G
                s = K[:n, kh, :] @ q[r * q_len + j, h] * scale
                p = np.exp(s - s.max())
                out[r * q_len + j, h] = (p / p.sum()) @ V[:n, kh, :]
    return out


# ---------------------------------------------------------------------------
# O7 KV overwrite — LLM-42 post, paragraph 3 (overwrite fast-path KV with the
# verifier's values at every verification)
# ---------------------------------------------------------------------------


def kv_overwrite(k_cache, v_cache, k_new, v_new, slots, block=16):
    """cache[slot[t]] <- (k_new[t], v_new[t]) for every t; other slots unchanged.
    Caches are modified in place (they are the oracle's own copies)."""
    for t, s in enumerate(np.asarray(slots, dtype=np.int64)):
        k_cache[s // block, :, s % block, :] = k_new[t]
        v_cache[s // block, :, s % block, :] = v_new[t]


# ---------------------------------------------------------------------------
# O6 Gumbel-max verification — Gumbel post (Gumbel-max trick; coupling:
# compare the draft token with the target token)
# ---------------------------------------------------------------------------


def perturbed_scores(logits32, noise32) -> np.ndarray:
    """s = fl32(logit + g): one IEEE fp32 addition, round to nearest even."""
    return np.asarray(logits32, dtype=np.float32) + np.asarray(noise32, dtype=np.float32)


def gumbel_verify(logits32, noise32, cand):
    """Coupled verification of K candidate tokens per request.

    logits32, noise32: [R, K, V] fp32; cand [R, K] int.
    target[r, j] = lowest index of the maximum of s (NaN never wins);
    accept[r]    = first j with target != cand, K if none;
    next[r]      = target[r, accept[r]], -1 if accept[r] == K.
    """
    s = perturbed_scores(logits32, noise32)
    s = np.where(np.isnan(s), np.float32(-np.inf), s)
    target = np.argmax(s, axis=-1).astype(np.int32)  # first occurrence of the max
    cand = np.asarray(cand)
    R, K = target.shape
    accept = np.full(R, K, dtype=np.int32)
    nxt = np.full(R, -1, dtype=np.int32)
    for r in range(R):
        for j in range(K):
            if target[r, j] != cand[r, j]:
                accept[r] = j
                nxt[r] = target[r, j]
                break
    return target, accept, nxt


def gumbel_topk(logits32, noise32, k):
    """Top-k of the perturbed scores (Gumbel post, Gumbel-max paragraph: top-k
    sampling comes out of the trick for free, with a pointer to "Stochastic
    Beams and Where to Find Them"): the k largest s = fl32(logit + g) of a row
    are k draws without replacement from the softmax.

    logits32, noise32: [..., V] fp32.  Returns (idx [..., k] int32, score
    [..., k] fp32): scores in descending order, equal scores in ascending
    index order; a NaN score counts as -inf (so it comes last).
    """
    s = perturbed_scores(logits32, noise32)
    s = np.where(np.isnan(s), np.float32(-np.inf), s)
    order = np.argsort(-s, axis=-1, kind="stable")[..., :k]  # stable: equal scores keep index order
    return order.astype(np.int32), np.take_along_axis(s, order, axis=-1)


def rollback(ctx, accept, nxt, cand):
    """Host bookkeeping after a verification (LLM-42 post, paragraph 3: roll
    back and fix).  Committed tokens: cand[:a] plus next (a < K); all K when
    a == K.  The verified context grows by min(a + 1, K); the new reference
    token is next (a < K) or cand[K-1] (a == K)."""
    K = np.asarray(cand).shape[1]
    new_ctx, committed, t0 = [], [], []
    for r in range(len(ctx)):
        a = int(accept[r])
        if a < K:
            toks = list(np.asarray(cand[r, :a])) + [int(nxt[r])]
        else:
            toks = list(np.asarray(cand[r, :K]))
        committed.append([int(t) for t in toks])
        new_ctx.append(int(ctx[r]) + min(a + 1, K))
        t0.append(int(toks[-1]))
    return np.asarray(new_ctx, dtype=np.int32), committed, np.asarray(t0, dtype=np.int32)


# ---------------------------------------------------------------------------
# O5 decoder forward over W = N*K tokens (LLM-42 post, paragraphs 3-4)
# ---------------------------------------------------------------------------


def decoder_forward(w, tokens, ctx, k_caches, v_caches, block_table, block=16):
    """Verifier forward.

    w: dict of fp64 weights — embed [V,H], lm_head [V,H], final_norm [H],
       layers: list of dicts (attn_norm, wq, wk, wv, wo, ffn_norm, w_gate,
       w_up, w_down), plus "shape" (a workloads.ModelShape).
    tokens [R, q_len]: input token of row (r, j) sits at position ctx[r] + j.
    k_caches / v_caches: per-layer fp64 caches [num_blocks, Hkv, block, D],
       modified in place: the rows' K/V are written before attention reads.
    Returns logits [R*q_len, V] (fp64).

    Layer: x += Wo * attn(rope(Wq n(x)), cache); x += Wd (silu(Wg n(x)) * Wu n(x));
    then logits = W_lm n(x).
    """
    sh = w["shape"]
    tokens = np.asarray(tokens)
    R, q_len = tokens.shape
    W = R * q_len
    H, Hq, Hkv, D = sh.hidden, sh.heads, sh.kv_heads, sh.head_dim
    pos = (np.asarray(ctx, dtype=np.int64)[:, None] + np.arange(q_len)[None, :]).reshape(-1)
    slots = np.array([int(block_table[t // q_len][int(p) // block]) * block + int(p) % block
                      for t, p in enumerate(pos)], dtype=np.int64)
    x = w["embed"][tokens.reshape(-1)].astype(np.float64)
    scale = 1.0 / np.sqrt(D)
    for li, L in enumerate(w["layers"]):
        h = rmsnorm(x, L["attn_norm"], sh.eps)
        q = rope(linear(h, L["wq"]).reshape(W, Hq, D), pos, sh.rope_theta)
        k = rope(linear(h, L["wk"]).reshape(W, Hkv, D), pos, sh.rope_theta)
        v = linear(h, L["wv"]).reshape(W, Hkv, D)
        kv_overwrite(k_caches[li], v_caches[li], k, v, slots, block)
        a = attention(q, k_caches[li], v_caches[li], block_table, ctx, q_len, scale, block)
        x = x + linear(a.reshape(W, Hq * D), L["wo"])
        h = rmsnorm(x, L["ffn_norm"], sh.eps)
        x = x + linear(silu(linear(h, L["w_gate"])) * linear(h, L["w_up"]), L["w_down"])
    return linear(rmsnorm(x, w["final_norm"], sh.eps), w["lm_head"])


def gumbel_sample(logits64, noise32):
    """Gumbel-max sample of one row: the logits are rounded once to fp32 (the
    verify rule is defined on fp32 logits) before s = fl32(logit + g)."""
    t, _, _ = gumbel_verify(np.asarray(logits64, dtype=np.float32)[None, None, :],
                            noise32[None, None, :], np.full((1, 1), -1))
    return int(t[0, 0])


def sequential_decode(w, t0, ctx, k_caches, v_caches, block_table, steps, noise_fn, block=16):
    """Reference decode, one token at a time (K = 1 per step).

    Request r starts from its last verified token t0[r] at position ctx[r].
    The token sampled for position p uses noise_fn(r, p) -> fp32 [V].
    Returns the generated tokens [R, steps] (positions ctx[r]+1 ..).
    """
    R = len(t0)
    cur = np.asarray(t0, dtype=np.int64).copy()
    c = np.asarray(ctx, dtype=np.int64).copy()
    out = np.zeros((R, steps), dtype=np.int32)
    for s in range(steps):
        logits = decoder_forward(w, cur[:, None], c, k_caches, v_caches, block_table, block)
        for r in range(R):
            out[r, s] = gumbel_sample(logits[r], noise_fn(r, int(c[r]) + 1))
        cur = out[:, s].astype(np.int64)
        c = c + 1
    return out


def dvr_decode(w, t0, ctx, k_caches, v_caches, block_table, n_tokens, K, drafter, noise_fn, block=16):
    """Decode-verify-rollback (LLM-42 post, paragraph 3) with Gumbel-coupled
    verification (Gumbel post).

    Each round: drafter(r, history, k) proposes K candidates; the verifier
    forward runs on [t0, c_0..c_{K-2}] at positions ctx..ctx+K-1; output j is
    sampled with the noise of position ctx+j+1 and compared with c_j; the
    accepted prefix plus the correction are committed (rollback()).  Returns
    the first n_tokens generated tokens per request [R, n_tokens].
    """
    R = len(t0)
    cur = np.asarray(t0, dtype=np.int32).copy()
    c = np.asarray(ctx, dtype=np.int32).copy()
    hist = [[] for _ in range(R)]
    while min(len(h) for h in hist) < n_tokens:
        cand = np.asarray([drafter(r, hist[r], K) for r in range(R)], dtype=np.int32)
        inp = np.concatenate([cur[:, None], cand[:, :K - 1]], axis=1)
        logits = decoder_forward(w, inp, c, k_caches, v_caches, block_table, block)
        V = logits.shape[-1]
        noise = np.stack([np.stack([noise_fn(r, int(c[r]) + j + 1) for j in range(K)]) for r in range(R)])
        _, acc, nxt = gumbel_verify(logits.astype(np.float32).reshape(R, K, V), noise, cand)
        c, committed, cur = rollback(c, acc, nxt, cand)
        for r in range(R):
            hist[r].extend(committed[r])
    return np.asarray([h[:n_tokens] for h in hist], dtype=np.int32)


# ---------------------------------------------------------------------------
# Tree verification by branches (Gumbel post: top-k drafts from the shared
# noise; with the noise fixed the output does not depend on the drafter).  A
# draft tree is given as B root-to-leaf chains per request; every chain is
# checked as an ordinary verifier row block on its own copy of the pages that
# hold positions L_r .. L_r+K-1.
# ---------------------------------------------------------------------------


def kv_copy_pages(k_cache, v_cache, src, dst):
    """Page dst[i] <- page src[i] of one layer's caches (every head, all 16
    slots, K and V), in place."""
    for s_, d_ in zip(src, dst):
        k_cache[d_] = k_cache[s_]
        v_cache[d_] = v_cache[s_]


def tree_select(accept, nxt):
    """accept, nxt [R, B]: per request the chain with the longest accepted
    prefix, the lowest chain index among equals.  Returns (best, accept, next) [R]."""
    accept = np.asarray(accept)
    nxt = np.asarray(nxt)
    R, B = accept.shape
    best = np.zeros(R, dtype=np.int32)
    for r in range(R):
        top = max(int(a) for a in accept[r])
        best[r] = min(b for b in range(B) if int(accept[r, b]) == top)
    rr = np.arange(R)
    return best, accept[rr, best].astype(np.int32), nxt[rr, best].astype(np.int32)


def tree_verify(w, t0, ctx, k_caches, v_caches, block_table, chains, private_pages, noise, block=16):
    """One tree verification.  chains [R, B, K]; private_pages [R, B-1, P]:
    chain b >= 1 of request r uses them in place of the request's pages from
    page ctx[r] // block on, the first receiving a copy of the request's page
    ctx[r] // block; noise [R, K, V] (one row per sampled position, shared by
    the chains).  Caches are modified in place (page copies, then each
    chain's K/V).  Returns (best, accept, next) [R] and the chains' targets
    [R, B, K]."""
    chains = np.asarray(chains)
    R, B, K = chains.shape
    bt = np.asarray(block_table)
    rows_bt = np.repeat(bt, B, axis=0).copy()
    src, dst = [], []
    for r in range(R):
        p0 = int(ctx[r]) // block
        n_pages = (int(ctx[r]) % block + K + block - 1) // block
        for b in range(1, B):
            pages = np.asarray(private_pages[r][b - 1])[:n_pages]
            rows_bt[r * B + b, p0:p0 + n_pages] = pages
            src.append(int(bt[r, p0]))
            dst.append(int(pages[0]))
    for li in range(len(k_caches)):
        kv_copy_pages(k_caches[li], v_caches[li], src, dst)
    t0s = np.repeat(np.asarray(t0), B)
    flat = chains.reshape(R * B, K)
    inp = np.concatenate([t0s[:, None], flat[:, :K - 1]], axis=1)
    logits = decoder_forward(w, inp, np.repeat(np.asarray(ctx), B), k_caches, v_caches, rows_bt, block)
    V = logits.shape[-1]
    nz = np.repeat(np.asarray(noise, dtype=np.float32)[:, None], B, axis=1).reshape(R * B, K, V)
    tgt, acc, nxt = gumbel_verify(logits.astype(np.float32).reshape(R * B, K, V), nz, flat)
    best, a, n = tree_select(acc.reshape(R, B), nxt.reshape(R, B))
    return best, a, n, tgt.reshape(R, B, K)
