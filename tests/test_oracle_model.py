"""Pins of the oracle's decoder forward, sequential decode and decode-verify-
rollback loop.

* A scalar-loop decoder (written here, independent of the oracle's vectorised
  code) on a micro model: same logits.
* Causality and KV handling: the K-token verifier forward gives the same
  logits as K one-token forwards (the verifier's own K/V is written before
  attention; rows see only earlier positions).
* Fast-path junk (even NaN) in the slots the verifier overwrites changes
  nothing (LLM-42 post, paragraph 3: overwrite the fast path's KV).
* Losslessness and drafter invariance (spec-dec guide: the target accepts only
  tokens it would write itself; Gumbel post: with a fixed seed the output does
  not depend on the drafter, or on whether one is used): DVR with several
  drafters reproduces the one-token-at-a-time decode exactly.
"""
import math

import numpy as np
import pytest

import oracle
import workloads as wl

MICRO = wl.ModelShape(layers=1, hidden=8, heads=2, kv_heads=1, head_dim=4, ffn=12, vocab=10,
                      rope_theta=10000.0)
SMALL = wl.ModelShape(layers=2, hidden=32, heads=4, kv_heads=2, head_dim=8, ffn=48, vocab=64,
                      rope_theta=10000.0)


def _weights64(shape, seed, std=0.3):
    w = wl.model_weights(shape, seed, "f32", std=std)
    d = dict(shape=shape, embed=w.embed.astype(np.float64), lm_head=w.lm_head.astype(np.float64),
             final_norm=w.final_norm.astype(np.float64), layers=[])
    for L in w.layers:
        d["layers"].append({k: v.astype(np.float64) for k, v in L.items()})
    return d


def _caches(shape, num_blocks, seed, fill=None):
    ks, vs = [], []
    for li in range(shape.layers):
        kc = wl.normal_f32(seed, (num_blocks, shape.kv_heads, 16, shape.head_dim), stream=(li, 0)).astype(np.float64)
        vc = wl.normal_f32(seed, (num_blocks, shape.kv_heads, 16, shape.head_dim), stream=(li, 1)).astype(np.float64)
        ks.append(kc)
        vs.append(vc)
    return ks, vs


def _scalar_decoder(w, tokens, ctx, kcs, vcs, bt):
    """Plain-loop reference for one request: python floats, explicit indices."""
    sh = w["shape"]
    H, Hq, Hkv, D, F, V = sh.hidden, sh.heads, sh.kv_heads, sh.head_dim, sh.ffn, sh.vocab
    G = Hq // Hkv

    def norm(x, g):
        ms = sum(v * v for v in x) / len(x)
        r = math.sqrt(ms + sh.eps)
        return [x[i] / r * g[i] for i in range(len(x))]

    def mv(M, x):
        return [sum(M[n][k] * x[k] for k in range(len(x))) for n in range(len(M))]

    def rot(vec, pos):
        half = D // 2
        out = list(vec)
        for i in range(half):
            ang = pos * sh.rope_theta ** (-2.0 * i / D)
            a, b = vec[i], vec[i + half]
            out[i] = a * math.cos(ang) - b * math.sin(ang)
            out[i + half] = b * math.cos(ang) + a * math.sin(ang)
        return out

    # per-layer key/value lists by absolute position (filled from the caches,
    # then overwritten by the new tokens, as the verifier does)
    n_tot = ctx + len(tokens)
    Ks = [[[list(kcs[l][bt[p // 16], h, p % 16]) for h in range(Hkv)] for p in range(n_tot)] for l in range(sh.layers)]
    Vs = [[[list(vcs[l][bt[p // 16], h, p % 16]) for h in range(Hkv)] for p in range(n_tot)] for l in range(sh.layers)]
    xs = [list(w["embed"][t]) for t in tokens]
    for l, L in enumerate(w["layers"]):
        qs = []
        for j, x in enumerate(xs):
            h = norm(x, L["attn_norm"])
            q = mv(L["wq"], h)
            k = mv(L["wk"], h)
            v = mv(L["wv"], h)
            pos = ctx + j
            qs.append([rot(q[hh * D:(hh + 1) * D], pos) for hh in range(Hq)])
            for hh in range(Hkv):
                Ks[l][pos][hh] = rot(k[hh * D:(hh + 1) * D], pos)
                Vs[l][pos][hh] = v[hh * D:(hh + 1) * D]
        new = []
        for j, x in enumerate(xs):
            att = []
            for hh in range(Hq):
                kv = hh // G
                n = ctx + j + 1
                sc = [sum(qs[j][hh][d] * Ks[l][p][kv][d] for d in range(D)) / math.sqrt(D) for p in range(n)]
                mx = max(sc)
                ex = [math.exp(s - mx) for s in sc]
                tot = sum(ex)
                att += [sum(ex[p] / tot * Vs[l][p][kv][d] for p in range(n)) for d in range(D)]
            o = mv(L["wo"], att)
            x = [x[i] + o[i] for i in range(H)]
            h = norm(x, L["ffn_norm"])
            gt = mv(L["w_gate"], h)
            up = mv(L["w_up"], h)
            act = [gt[i] / (1 + math.exp(-gt[i])) * up[i] for i in range(F)]
            dn = mv(L["w_down"], act)
            new.append([x[i] + dn[i] for i in range(H)])
        xs = new
    return [mv(w["lm_head"], norm(x, w["final_norm"])) for x in xs]


def test_decoder_matches_scalar_loop_micro():
    w = _weights64(MICRO, 1)
    ctx, q_len = 19, 3
    lay = wl.paged_layout([ctx], q_len, seed=2)
    kcs, vcs = _caches(MICRO, lay.num_blocks, 3)
    toks = np.array([[3, 7, 1]])
    ref = _scalar_decoder(w, list(toks[0]), ctx, [k.copy() for k in kcs], [v.copy() for v in vcs],
                          lay.block_table[0])
    got = oracle.decoder_forward(w, toks, [ctx], kcs, vcs, lay.block_table)
    np.testing.assert_allclose(got, np.asarray(ref), rtol=1e-11, atol=1e-12)


def test_verify_forward_equals_one_token_forwards_and_overwrites_junk():
    """K-token verifier forward == K one-token forwards (causality + KV written
    before attention).  NaN junk in the fast-path slots changes nothing."""
    sh = SMALL
    w = _weights64(sh, 4)
    ctx = [40, 17, 63]
    K = 4
    lay = wl.paged_layout(ctx, K, seed=5)
    kcs, vcs = _caches(sh, lay.num_blocks, 6)
    slots = lay.slots()
    junk_k = [k.copy() for k in kcs]
    junk_v = [v.copy() for v in vcs]
    for li in range(sh.layers):
        for s in slots:
            junk_k[li][s // 16, :, s % 16] = np.nan
            junk_v[li][s // 16, :, s % 16] = np.nan
    toks = wl.tokens(7, (3, K), sh.vocab)
    a = oracle.decoder_forward(w, toks, ctx, junk_k, junk_v, lay.block_table)
    assert np.isfinite(a).all()
    kc1 = [k.copy() for k in kcs]
    vc1 = [v.copy() for v in vcs]
    rows = []
    for j in range(K):
        rows.append(oracle.decoder_forward(w, toks[:, j:j + 1], np.asarray(ctx) + j, kc1, vc1, lay.block_table))
    b = np.stack(rows, axis=1).reshape(3 * K, -1)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)
    # a row's logits do not depend on later candidates
    toks2 = toks.copy()
    toks2[:, 2:] = (toks2[:, 2:] + 5) % sh.vocab
    c = oracle.decoder_forward(w, toks2, ctx, [k.copy() for k in kcs], [v.copy() for v in vcs], lay.block_table)
    np.testing.assert_array_equal(c.reshape(3, K, -1)[:, :2], a.reshape(3, K, -1)[:, :2])


def _noise_fn(seed, V):
    cache = {}

    def f(r, p):
        if (r, p) not in cache:
            cache[(r, p)] = wl.gumbel_noise(seed, [r], [p], V)[0]
        return cache[(r, p)]

    return f


@pytest.mark.parametrize("K", [1, 3, 4])
def test_dvr_is_lossless_and_drafter_invariant(K):
    """DVR output == sequential decode for a perfect, an always-wrong, a random
    and a half-right drafter (spec-dec guide: lossless; Gumbel post: drafter
    invariance at a fixed seed)."""
    sh = SMALL
    w = _weights64(sh, 8, std=0.5)  # sharper logits -> repeated tokens are likely
    ctx = [20, 33]
    n = 10
    lay = wl.paged_layout(ctx, n + K + 1, seed=9)
    kcs, vcs = _caches(sh, lay.num_blocks, 10)
    t0 = np.array([5, 11])
    noise = _noise_fn(11, sh.vocab)
    seq = oracle.sequential_decode(w, t0, ctx, [k.copy() for k in kcs], [v.copy() for v in vcs],
                                   lay.block_table, n + K, noise)
    g = wl.rng(12)
    drafters = {
        "perfect": lambda r, h, k: [int(t) for t in seq[r, len(h):len(h) + k]],
        "wrong": lambda r, h, k: [(int(t) + 1) % sh.vocab for t in seq[r, len(h):len(h) + k]],
        "random": lambda r, h, k: [int(t) for t in g.integers(0, sh.vocab, size=k)],
        "half": lambda r, h, k: [int(t) if i < k // 2 else 0 for i, t in enumerate(seq[r, len(h):len(h) + k])],
    }
    for name, dr in drafters.items():
        out = oracle.dvr_decode(w, t0, ctx, [k.copy() for k in kcs], [v.copy() for v in vcs],
                                lay.block_table, n, K, dr, noise)
        np.testing.assert_array_equal(out, seq[:, :n], err_msg=name)


def _tree_world(sh, ctx, K, B, seed):
    """Requests with random-KV contexts, their block tables (covering
    L_r .. L_r+K-1) and (B-1) x 2 spare pages per request for the chains."""
    lay = wl.paged_layout(ctx, K, seed=seed)
    R = len(ctx)
    n_priv = 2 * max(B - 1, 1)
    nb = lay.num_blocks + R * n_priv
    kcs, vcs = _caches(sh, nb, seed + 1)
    priv = (lay.num_blocks + np.arange(R * n_priv)).reshape(R, n_priv)[:, :2 * (B - 1)].reshape(R, B - 1, 2)
    return lay, kcs, vcs, priv


def _seq_tokens(w, t0, ctx, kcs, vcs, bt, K, noise):
    return oracle.sequential_decode(w, t0, ctx, [k.copy() for k in kcs], [v.copy() for v in vcs], bt, K, noise)


def test_tree_of_every_chain_accepts_the_decode():
    """Tree verification over ALL V^K chains of a micro vocabulary: exactly one
    chain is the target's own continuation, so every request accepts all K
    tokens, and the selected chain equals one-token-at-a-time decoding (spec-dec
    guide: the target accepts only what it would write itself).  A wrong page
    copy, a chain mixed up with another or a wrong selection fails this."""
    sh = MICRO
    K = 2
    w = _weights64(sh, 21, std=0.6)
    ctx = [13, 30]  # page offsets 13 and 14: positions L .. L+K-1 cross into the next page for r = 1 only
    chains_one = np.array([[a, b] for a in range(sh.vocab) for b in range(sh.vocab)], dtype=np.int32)
    B = len(chains_one)
    lay, kcs, vcs, priv = _tree_world(sh, ctx, K, B, 22)
    noise_fn = _noise_fn(23, sh.vocab)
    t0 = np.array([4, 7])
    noise = np.stack([np.stack([noise_fn(r, ctx[r] + j + 1) for j in range(K)]) for r in range(2)])
    seq = _seq_tokens(w, t0, ctx, kcs, vcs, lay.block_table, K, noise_fn)
    chains = np.stack([chains_one, chains_one])
    best, acc, nxt, tgt = oracle.tree_verify(w, t0, ctx, kcs, vcs, lay.block_table, chains, priv, noise)
    np.testing.assert_array_equal(acc, [K, K])
    np.testing.assert_array_equal(nxt, [-1, -1])
    for r in range(2):
        np.testing.assert_array_equal(chains[r, best[r]], seq[r, :K])
        # every chain's first target is the decode's first token (shared noise row)
        assert (tgt[r, :, 0] == seq[r, 0]).all()


def test_tree_commits_the_decode_prefix_of_its_best_chain():
    """Random chains plus chains that follow the decode for d tokens and then
    differ: the accepted length is the longest such d, the selected chain the
    first chain reaching it, and accepted tokens + correction are the decode's
    first d + 1 tokens (Gumbel post: the output does not depend on the
    drafter)."""
    sh = SMALL
    K, B = 4, 5
    w = _weights64(sh, 24, std=0.5)
    ctx = [29, 16, 45]
    lay, kcs, vcs, priv = _tree_world(sh, ctx, K, B, 25)
    noise_fn = _noise_fn(26, sh.vocab)
    t0 = np.array([3, 9, 17])
    R = len(ctx)
    noise = np.stack([np.stack([noise_fn(r, ctx[r] + j + 1) for j in range(K)]) for r in range(R)])
    seq = _seq_tokens(w, t0, ctx, kcs, vcs, lay.block_table, K, noise_fn)
    g = wl.rng(27)
    chains = g.integers(0, sh.vocab, size=(R, B, K)).astype(np.int32)
    plan = [(1, 2, 3), (0, 0, 0), (3, 1, 3)]  # per request: d of chains 1, 2 and of chain 4 (a duplicate d)
    for r, (d1, d2, d4) in enumerate(plan):
        for b, d in ((1, d1), (2, d2), (4, d4)):
            chains[r, b, :d] = seq[r, :d]
            if d < K:
                chains[r, b, d] = (seq[r, d] + 1) % sh.vocab
        for b in (0, 3):  # random chains may not follow the decode at all
            if chains[r, b, 0] == seq[r, 0]:
                chains[r, b, 0] = (seq[r, 0] + 2) % sh.vocab
    best, acc, nxt, _ = oracle.tree_verify(w, t0, ctx, kcs, vcs, lay.block_table, chains, priv, noise)
    np.testing.assert_array_equal(acc, [3, 0, 3])
    np.testing.assert_array_equal(best, [4, 0, 1])
    for r in range(R):
        a = int(acc[r])
        committed = list(chains[r, best[r], :a]) + ([int(nxt[r])] if a < K else [])
        np.testing.assert_array_equal(committed, seq[r, :len(committed)])


def test_tree_select_ties_go_to_the_lowest_chain():
    acc = np.array([[2, 4, 4, 1], [0, 0, 0, 0], [3, 1, 3, 3]])
    nxt = np.arange(12).reshape(3, 4)
    best, a, n = oracle.tree_select(acc, nxt)
    np.testing.assert_array_equal(best, [1, 0, 0])
    np.testing.assert_array_equal(a, [4, 0, 3])
    np.testing.assert_array_equal(n, [1, 4, 8])
