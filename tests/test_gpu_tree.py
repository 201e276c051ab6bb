"""Tree verification by branches on the GPU (Gumbel post: top-k drafts from
the shared noise, and at a fixed seed the output does not depend on the
drafter; LLM-42 post, paragraph 3: the verifier's K/V replaces the fast
path's).

* kv_copy_pages: whole-page bit copies, skipped pairs left alone;
* tree_select: longest accepted prefix, lowest chain among equals, against
  the oracle;
* a tree of B chains per request on the tiny fp32 decoder: decisions equal
  the oracle's tree verification, the selected chain's targets and K/V equal,
  bit for bit, the same chain verified on its own with the request's own
  pages, and accepted tokens + correction are one-token-at-a-time decoding;
  after the request adopts its selected chain's pages, the next verifier
  round gives the same bits as after the single-chain round.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_util import DEV, announce, bits, dev_i32, sync

pytestmark = pytest.mark.gpu

TINY = wl.TINY


@pytest.fixture(scope="module")
def biv():
    import invariant_verify_verifier_amd as m

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_kv_copy_pages_bitwise(biv, dtype):
    nb, Hkv, D = 40, 8, 128
    g = torch.Generator(device="cpu").manual_seed(5)
    k = torch.randn((nb, Hkv, 16, D), generator=g).to(dtype)
    v = torch.randn((nb, Hkv, 16, D), generator=g).to(dtype)
    src = [3, 7, 0, 12, 39, 50, 5]
    dst = [20, 21, 33, 34, 35, 36, 5]  # 50: outside the cache; 5 -> 5: both skipped
    want_k, want_v = k.clone(), v.clone()
    for s_, d_ in zip(src, dst):
        if 0 <= s_ < nb and 0 <= d_ < nb and s_ != d_:
            want_k[d_] = k[s_]
            want_v[d_] = v[s_]
    kd, vd = k.to(DEV), v.to(DEV)
    announce("kv_copy_pages", dtype)
    biv.kv_copy_pages(dev_i32(src), dev_i32(dst), kd, vd)
    sync()
    assert np.array_equal(bits(kd), bits(want_k)) and np.array_equal(bits(vd), bits(want_v))


def test_tree_select_matches_oracle(biv):
    g = wl.rng(40)
    for R, B in ((1, 1), (7, 3), (64, 16), (300, 5)):
        acc = g.integers(0, 5, size=(R, B)).astype(np.int32)
        nxt = g.integers(-1, 1000, size=(R, B)).astype(np.int32)
        best = torch.empty(R, dtype=torch.int32, device=DEV)
        a = torch.empty_like(best)
        n = torch.empty_like(best)
        announce("tree_select", R, B)
        biv.tree_select(dev_i32(acc), dev_i32(nxt), best, a, n)
        sync()
        ob, oa, on = oracle.tree_select(acc, nxt)
        assert np.array_equal(best.cpu().numpy(), ob)
        assert np.array_equal(a.cpu().numpy(), oa) and np.array_equal(n.cpu().numpy(), on)


def _oracle_weights(w):
    d = dict(shape=w.shape, embed=oracle.as_f64(w.embed, w.dtype), lm_head=oracle.as_f64(w.lm_head, w.dtype),
             final_norm=oracle.as_f64(w.final_norm, w.dtype), layers=[])
    for L in w.layers:
        d["layers"].append({k: oracle.as_f64(v, w.dtype) for k, v in L.items()})
    return d


def test_tree_verify_tiny_matches_oracle_and_single_chains(biv):
    from invariant_verify_verifier_amd import verifier as V

    K, B = 4, 4
    ctx = np.array([45, 61, 96], np.int32)  # 45 + 4 and 61 + 4 cross a page boundary
    R = len(ctx)
    w = wl.model_weights(TINY, wl.SEEDS["tiny_weights"], "f32")
    ow = _oracle_weights(w)
    model = V.VerifierModel.from_host(w, max_pos=1024)
    lay = wl.paged_layout(ctx, 2 * K, seed=41)  # room for a second round
    priv = (lay.num_blocks + np.arange(R * (B - 1) * 2)).reshape(R, B - 1, 2).astype(np.int32)
    nb = lay.num_blocks + priv.size
    kc = [wl.normal_f32(42, (nb, TINY.kv_heads, 16, TINY.head_dim), stream=(li, 0)) for li in range(TINY.layers)]
    vc = [wl.normal_f32(42, (nb, TINY.kv_heads, 16, TINY.head_dim), stream=(li, 1)) for li in range(TINY.layers)]
    t0 = wl.tokens(43, (R,), TINY.vocab)
    nseed = 44
    noise = wl.gumbel_noise(nseed, np.repeat(np.arange(R), K).reshape(R, K), ctx[:, None] + np.arange(K) + 1,
                            TINY.vocab)
    nf = lambda r, p: wl.gumbel_noise(nseed, [r], [p], TINY.vocab)[0]
    seq = oracle.sequential_decode(ow, t0, ctx, [k.astype(np.float64) for k in kc], [v.astype(np.float64) for v in vc],
                                   lay.block_table, K, nf)
    # chains: 0 random (first token off the decode), 1 and 2 follow the decode
    # for d1 < d2 tokens, 3 repeats chain 2 (the tie goes to chain 2)
    g = wl.rng(45)
    chains = g.integers(0, TINY.vocab, size=(R, B, K)).astype(np.int32)
    plan = [(1, 3), (0, 2), (2, 4)]
    for r, (d1, d2) in enumerate(plan):
        chains[r, 0, 0] = (seq[r, 0] + 1) % TINY.vocab
        for b, d in ((1, d1), (2, d2)):
            chains[r, b, :d] = seq[r, :d]
            if d < K:
                chains[r, b, d] = (seq[r, d] + 7) % TINY.vocab
        chains[r, 3] = chains[r, 2]
    ob, oa, on, _ = oracle.tree_verify(ow, t0, ctx, [k.astype(np.float64) for k in kc],
                                       [v.astype(np.float64) for v in vc], lay.block_table, chains, priv, noise)
    assert np.array_equal(oa, [3, 2, 4]) and np.array_equal(ob, [2, 2, 2])

    def caches():
        return [(torch.from_numpy(k).to(DEV), torch.from_numpy(v).to(DEV)) for k, v in zip(kc, vc)]

    cs = caches()
    tb = V.make_tree_batch(t0, chains, ctx, lay.block_table, priv, noise)
    announce("tree verify tiny", R, B, K)
    best, acc, nxt, tgt = V.verify_tree(model, tb, cs)
    sync()
    best, acc, nxt = best.cpu().numpy(), acc.cpu().numpy(), nxt.cpu().numpy()
    assert np.array_equal(best, ob) and np.array_equal(acc, oa) and np.array_equal(nxt, on)
    for r in range(R):
        a = int(acc[r])
        committed = list(chains[r, best[r], :a]) + ([int(nxt[r])] if a < K else [])
        assert np.array_equal(committed, seq[r, :len(committed)]), f"request {r}"
    tree_tgt = tgt.cpu().numpy().reshape(R, B, K)
    # the selected chain alone, on the request's own pages: the same bits
    cs1 = caches()
    one = V.make_batch(t0, chains[np.arange(R), best], ctx, lay.block_table,
                       np.ascontiguousarray(noise, dtype=np.float32))
    announce("tree verify: selected chains alone")
    _, t1, a1, n1 = model.verify(one, cs1)
    sync()
    assert np.array_equal(t1.cpu().numpy(), tree_tgt[np.arange(R), best])
    assert np.array_equal(a1.cpu().numpy(), acc) and np.array_equal(n1.cpu().numpy(), nxt)
    for r in range(R):
        b = int(best[r])
        p0 = int(ctx[r]) // 16
        for j in range(K):
            p = int(ctx[r]) + j
            own = int(lay.block_table[r, p // 16])
            mine = own if b == 0 else int(priv[r, b - 1, p // 16 - p0])
            for li in range(TINY.layers):
                for t in (0, 1):
                    assert np.array_equal(bits(cs[li][t][mine, :, p % 16]), bits(cs1[li][t][own, :, p % 16])), \
                        f"request {r} position {p} layer {li}"
        if b > 0:  # the context rows of the copied page
            own0, mine0 = int(lay.block_table[r, p0]), int(priv[r, b - 1, 0])
            for li in range(TINY.layers):
                for t, src in ((0, kc), (1, vc)):
                    got = bits(cs[li][t][mine0, :, :int(ctx[r]) % 16])
                    assert np.array_equal(got, bits(torch.from_numpy(src[li][own0, :, :int(ctx[r]) % 16])))

    # next round: the request adopts the selected chain's pages; the round
    # after it must see the same K/V as after the single-chain round
    new_bt, _ = V.adopt_chain_pages(lay.block_table, ctx, best, priv, K)
    ctx2, _, t02 = V.rollback(ctx, acc, nxt, chains[np.arange(R), best])
    cand2 = wl.tokens(46, (R, K), TINY.vocab)
    noise2 = wl.gumbel_noise(nseed, np.repeat(np.arange(R), K).reshape(R, K), ctx2[:, None] + np.arange(K) + 1,
                             TINY.vocab)
    announce("tree verify: second round after adopting pages")
    _, ta, aa, na = model.verify(V.make_batch(t02, cand2, ctx2, new_bt, noise2), cs)
    ta, aa, na = ta.cpu().numpy(), aa.cpu().numpy(), na.cpu().numpy()
    _, tb_, ab, nb_ = model.verify(V.make_batch(t02, cand2, ctx2, lay.block_table, noise2), cs1)
    sync()
    assert np.array_equal(ta, tb_.cpu().numpy()) and np.array_equal(aa, ab.cpu().numpy())
    assert np.array_equal(na, nb_.cpu().numpy())
