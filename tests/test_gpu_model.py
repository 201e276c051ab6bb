"""End-to-end verifier step on the GPU.

Tiny fp32 decoder (2 layers, hidden 256, 4 heads x 64, FFN 1024, vocab 4096,
N = 4 requests x K = 4 candidates, 128-token prompts):
  * logits within fp32 tolerance of the oracle, verify decisions bit-exact,
    planted first divergence recovered exactly;
  * batch invariance at 1..16 co-batched requests, bitwise;
  * lossless, drafter-invariant DVR on the GPU: the verify-rollback loop
    reproduces one-token-at-a-time decoding bit for bit for several drafters
    (LLM-42 post, paragraph 3; Gumbel post, drafter invariance).
Llama-3-8B-shaped slice (2 of the 32 layers, 4 requests, contexts ~2048, K=8,
bf16): logits vs the oracle, planted divergence, subset invariance.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_util import DEV, announce, bits, dev_i32, f64, sync
from storage_model import bf16_storage_forward, error_bound
from tolerances import check_f32

pytestmark = pytest.mark.gpu

TINY = wl.TINY
K_TINY = 4


@pytest.fixture(scope="module")
def V():
    import invariant_verify_verifier_amd.verifier as verifier

    assert torch.cuda.is_available()
    return verifier


def _oracle_weights(w):
    d = dict(shape=w.shape, embed=oracle.as_f64(w.embed, w.dtype), lm_head=oracle.as_f64(w.lm_head, w.dtype),
             final_norm=oracle.as_f64(w.final_norm, w.dtype), layers=[])
    for L in w.layers:
        d["layers"].append({k: oracle.as_f64(v, w.dtype) for k, v in L.items()})
    return d


def _noise(seed, V, reqs, positions):
    return wl.gumbel_noise(seed, reqs, positions, V)


class TinyWorld:
    """16 requests with 128-token prompts prefilled on the GPU (one request at
    a time, the fixed-batch prefill the LLM-42 post relies on) and on the
    oracle; the first generated token t0 comes from the oracle."""

    def __init__(self, V, n_req=16, extra=64):
        self.w = wl.model_weights(TINY, wl.SEEDS["tiny_weights"], "f32")
        self.ow = _oracle_weights(self.w)
        self.model = V.VerifierModel.from_host(self.w, max_pos=4096)
        self.n = n_req
        self.prompts = wl.tokens(wl.SEEDS["tiny_prompt"], (n_req, 128), TINY.vocab)
        self.ctx0 = np.full(n_req, 128, np.int32)
        self.lay = wl.paged_layout(np.zeros(n_req, np.int32), 128 + extra, seed=5)
        self.caches = self.model.alloc_kv(self.lay.num_blocks)
        nb = self.lay.num_blocks
        self.okc = [np.zeros((nb, TINY.kv_heads, 16, TINY.head_dim)) for _ in range(TINY.layers)]
        self.ovc = [np.zeros((nb, TINY.kv_heads, 16, TINY.head_dim)) for _ in range(TINY.layers)]
        self.t0 = np.zeros(n_req, np.int32)
        for r in range(n_req):
            bt = self.lay.block_table[r:r + 1]
            toks = self.prompts[r]
            pos = np.arange(128, dtype=np.int32)
            slots = (bt[0, pos // 16].astype(np.int64) * 16 + pos % 16)
            announce("tiny prefill", r)
            self.model.forward(dev_i32(toks), dev_i32(pos), dev_i32([0]), 128, dev_i32(bt),
                               torch.from_numpy(slots).to(DEV), self.caches)
            lg = oracle.decoder_forward(self.ow, toks[None, :], [0], self.okc, self.ovc, self.lay.block_table[r:r + 1])
            g = _noise(wl.SEEDS["tiny_noise"], TINY.vocab, [r], [128])[0]
            self.t0[r] = oracle.gumbel_sample(lg[-1], g)
        sync()

    def noise_fn(self):
        cache = {}

        def f(r, p):
            if (r, p) not in cache:
                cache[(r, p)] = _noise(wl.SEEDS["tiny_noise"], TINY.vocab, [r], [p])[0]
            return cache[(r, p)]

        return f

    def batch(self, V, reqs, cand, ctx=None):
        reqs = np.asarray(reqs)
        ctx = self.ctx0[reqs] if ctx is None else np.asarray(ctx)
        K = cand.shape[1]
        pos = ctx[:, None] + np.arange(K)[None, :] + 1
        nz = _noise(wl.SEEDS["tiny_noise"], TINY.vocab, np.repeat(reqs, K).reshape(-1, K), pos)
        return V.make_batch(self.t0[reqs], cand, ctx, self.lay.block_table[reqs], nz)


@pytest.fixture(scope="module")
def tiny(V):
    return TinyWorld(V)


def _oracle_seq(tiny, reqs, steps):
    okc = [k.copy() for k in tiny.okc]
    ovc = [v.copy() for v in tiny.ovc]
    reqs = np.asarray(reqs)
    nf = tiny.noise_fn()
    return oracle.sequential_decode(tiny.ow, tiny.t0[reqs], tiny.ctx0[reqs], okc, ovc, tiny.lay.block_table[reqs],
                                    steps, lambda r, p: nf(int(reqs[r]), p))


def test_tiny_verify_parity_and_planted_divergence(V, tiny):
    reqs = np.arange(4)
    K = K_TINY
    seq = _oracle_seq(tiny, reqs, K)
    d = wl.rng(wl.SEEDS["tiny_plant"]).integers(0, K, size=4)
    cand = wl.plant_divergence(seq, d, TINY.vocab, wl.SEEDS["tiny_plant"])
    b = tiny.batch(V, reqs, cand)
    announce("tiny verify")
    logits, tgt, acc, nxt = tiny.model.verify(b, tiny.caches)
    sync()
    # oracle verify forward on the same inputs
    okc = [k.copy() for k in tiny.okc]
    ovc = [v.copy() for v in tiny.ovc]
    toks = np.concatenate([tiny.t0[reqs, None], cand[:, :K - 1]], axis=1)
    olog = oracle.decoder_forward(tiny.ow, toks, tiny.ctx0[reqs], okc, ovc, tiny.lay.block_table[reqs])
    err = check_f32(f64(logits), olog, axis=1, what="tiny logits")
    noise = b.noise.cpu().numpy().reshape(4, K, -1)
    t_ref, a_ref, n_ref = oracle.gumbel_verify(olog.astype(np.float32).reshape(4, K, -1), noise, cand)
    s = oracle.perturbed_scores(olog.astype(np.float32).reshape(4, K, -1), noise)
    top2 = np.sort(s, axis=-1)[..., -2:]
    print(f"tiny: logits rel err {err:.2e}; min top-2 margin of s {np.min(top2[..., 1] - top2[..., 0]):.3e}")
    assert np.array_equal(tgt.cpu().numpy(), t_ref)
    assert np.array_equal(acc.cpu().numpy(), d) and np.array_equal(a_ref, d)
    assert np.array_equal(nxt.cpu().numpy(), n_ref)
    # the decision on the GPU's own logits is the oracle's rule, bit for bit
    t2, a2, n2 = oracle.gumbel_verify(f64(logits).astype(np.float32).reshape(4, K, -1), noise, cand)
    assert np.array_equal(tgt.cpu().numpy(), t2)


def test_tiny_batch_invariance_1_to_16(V, tiny):
    """Each request's logits are bit-identical whether verified alone or with
    up to 15 other requests, in any order."""
    K = K_TINY
    g = wl.rng(77)
    cand_all = g.integers(0, TINY.vocab, size=(tiny.n, K)).astype(np.int32)
    b = tiny.batch(V, np.arange(tiny.n), cand_all)
    announce("tiny invariance full batch")
    full = bits(tiny.model.verify(b, tiny.caches)[0]).reshape(tiny.n, K, -1).copy()
    for size in range(1, tiny.n + 1):
        reqs = g.permutation(tiny.n)[:size]
        bb = tiny.batch(V, reqs, cand_all[reqs])
        announce("tiny invariance size", size)
        got = bits(tiny.model.verify(bb, tiny.caches)[0]).reshape(size, K, -1)
        for i, r in enumerate(reqs):
            assert np.array_equal(got[i], full[r]), f"request {r} changed in a batch of {size}"


def _gpu_sequential(V, tiny, reqs, steps):
    """One token per step (K = 1) for all requests in `reqs`, on the GPU."""
    reqs = np.asarray(reqs)
    cur = tiny.t0[reqs].copy()
    ctx = tiny.ctx0[reqs].copy()
    out = np.zeros((len(reqs), steps), np.int32)
    for s in range(steps):
        b = tiny.batch(V, reqs, np.zeros((len(reqs), 1), np.int32), ctx=ctx)
        b.tokens.copy_(torch.from_numpy(cur).to(DEV))
        _, tgt, _, _ = tiny.model.verify(b, tiny.caches)
        out[:, s] = tgt.cpu().numpy()[:, 0]
        cur = out[:, s].copy()
        ctx = ctx + 1
    return out


def _gpu_dvr(V, tiny, reqs, n, K, drafter):
    reqs = np.asarray(reqs)
    t0 = tiny.t0[reqs].copy()
    ctx = tiny.ctx0[reqs].copy()
    hist = [[] for _ in reqs]
    while min(len(h) for h in hist) < n:
        cand = np.asarray([drafter(i, hist[i], K) for i in range(len(reqs))], np.int32)
        pos = ctx[:, None] + np.arange(K)[None, :] + 1
        nz = _noise(wl.SEEDS["tiny_noise"], TINY.vocab, np.repeat(reqs, K).reshape(-1, K), pos)
        b = V.make_batch(t0, cand, ctx, tiny.lay.block_table[reqs], nz)
        _, _, acc, nxt = tiny.model.verify(b, tiny.caches)
        ctx, committed, t0 = V.rollback(ctx, acc.cpu().numpy(), nxt.cpu().numpy(), cand)
        for i in range(len(reqs)):
            hist[i].extend(committed[i])
    return np.asarray([h[:n] for h in hist], np.int32)


def test_tiny_dvr_equals_sequential_decode_on_gpu(V, tiny):
    reqs = np.arange(4)
    n, K = 12, K_TINY
    announce("tiny gpu sequential decode")
    seq = _gpu_sequential(V, tiny, reqs, n + K)
    oseq = _oracle_seq(tiny, reqs, n)
    assert np.array_equal(seq[:, :n], oseq), "GPU sequential decode differs from the oracle's"
    g = wl.rng(5)
    drafters = {
        "perfect": lambda i, h, k: [int(t) for t in seq[i, len(h):len(h) + k]],
        "wrong": lambda i, h, k: [(int(t) + 1) % TINY.vocab for t in seq[i, len(h):len(h) + k]],
        "random": lambda i, h, k: [int(t) for t in g.integers(0, TINY.vocab, size=k)],
        "half": lambda i, h, k: [int(t) if j < k // 2 else 0 for j, t in enumerate(seq[i, len(h):len(h) + k])],
    }
    for name, dr in drafters.items():
        announce("tiny gpu dvr", name)
        out = _gpu_dvr(V, tiny, reqs, n, K, dr)
        assert np.array_equal(out, seq[:, :n]), name


# ---------------------------------------------------------------------------
# Llama-3-8B-shaped slice
# ---------------------------------------------------------------------------

SLICE_LAYERS = 2
# Ceiling on the derived max-error bound of the slice (1.5 x the precision
# model's max distance from fp64, ~0.053 here): a bound above it would mean the
# model or the oracle changed.
SLICE_LOGIT_ABS_CEIL = 0.1


def _slice_world(V, ctx, seed=40):
    sh = wl.LLAMA3_8B
    dw = wl.device_model_weights(sh, seed, layers=SLICE_LAYERS)
    shape = V.Shape(SLICE_LAYERS, sh.hidden, sh.heads, sh.kv_heads, sh.head_dim, sh.ffn, sh.vocab, sh.eps,
                    sh.rope_theta)
    model = V.VerifierModel(shape, torch.bfloat16, dw["layers"], dw["embed"], dw["lm_head"], dw["final_norm"],
                            max_pos=16384)
    lay = wl.paged_layout(ctx, 8, seed=seed + 2, spare_blocks=5)
    caches = wl.device_kv_cache(sh, lay.num_blocks, seed + 1, layers=SLICE_LAYERS)
    return sh, dw, model, lay, caches


def _slice_oracle_weights(sh, dw):
    H, D, F = sh.hidden, sh.head_dim, sh.ffn
    q, kv = sh.heads * D, sh.kv_heads * D
    c = lambda t: f64(t)
    d = dict(shape=wl.ModelShape(SLICE_LAYERS, H, sh.heads, sh.kv_heads, D, F, sh.vocab, sh.eps, sh.rope_theta),
             embed=c(dw["embed"]), lm_head=c(dw["lm_head"]), final_norm=c(dw["final_norm"]), layers=[])
    for L in dw["layers"]:
        wqkv, wgu = c(L["wqkv"]), c(L["w_gu"])
        d["layers"].append(dict(attn_norm=c(L["attn_norm"]), wq=wqkv[:q], wk=wqkv[q:q + kv], wv=wqkv[q + kv:],
                                wo=c(L["wo"]), ffn_norm=c(L["ffn_norm"]), w_gate=wgu[:F], w_up=wgu[F:],
                                w_down=c(L["w_down"])))
    return d


def test_llama8b_slice_parity_planted_and_invariance(V):
    sh = wl.LLAMA3_8B
    R, K = 4, 8
    ctx = wl.context_lengths(42, R, 1800, 2300)
    announce("8b slice setup", list(ctx))
    _, dw, model, lay, caches = _slice_world(V, ctx)
    okc = [f64(k) for k, _ in caches]
    ovc = [f64(v) for _, v in caches]
    toks_cand = wl.tokens(43, (R, K), sh.vocab)
    t0 = wl.tokens(44, (R,), sh.vocab)
    pos = ctx[:, None] + np.arange(K)[None, :] + 1
    nz = wl.gumbel_noise(45, np.repeat(np.arange(R), K).reshape(R, K), pos, sh.vocab)
    b = V.make_batch(t0, toks_cand, ctx, lay.block_table, nz)
    announce("8b slice verify")
    logits, tgt, _, _ = model.verify(b, caches)
    sync()
    g_logits = f64(logits).copy()
    g_tgt = tgt.cpu().numpy().copy()
    # every row: the oracle's verify rule on the step's own fp32 logits gives its targets bit for bit
    r_tgt, _, _ = oracle.gumbel_verify(g_logits.astype(np.float32).reshape(R, K, -1), nz, toks_cand)
    assert np.array_equal(g_tgt, r_tgt)
    # oracle and the bf16 precision model on the same inputs (their own
    # copies of the pre-pass caches)
    ow = _slice_oracle_weights(sh, dw)
    toks = np.concatenate([t0[:, None], toks_cand[:, :K - 1]], axis=1)
    mkc = [c.copy() for c in okc]
    mvc = [c.copy() for c in ovc]
    olog = oracle.decoder_forward(ow, toks, ctx, okc, ovc, lay.block_table)
    mlog = bf16_storage_forward(ow, toks, ctx, mkc, mvc, lay.block_table)
    err = np.abs(g_logits - olog)
    rms_b, max_b = error_bound(mlog, olog)
    rms = float(np.sqrt(np.mean(err * err)))
    print(f"8b slice: |step - fp64| max {err.max():.4f} rms {rms:.5f}; model max "
          f"{np.abs(mlog - olog).max():.4f}; bounds rms {rms_b:.5f} max {max_b:.4f}; |ref| max {np.abs(olog).max():.2f}")
    assert rms <= rms_b and err.max() <= max_b <= SLICE_LOGIT_ABS_CEIL
    bound = max_b
    s = oracle.perturbed_scores(olog.astype(np.float32).reshape(R, K, -1), nz)
    t_ref = np.argmax(s, axis=-1)
    srt = np.sort(s, axis=-1)
    margin = srt[..., -1] - srt[..., -2]
    safe = margin > 2 * bound + 1e-5  # within the bound, such a row cannot change its argmax
    print(f"8b slice: {int((~safe).sum())} of {R * K} rows within twice the derived bound of a tie")
    assert np.array_equal(g_tgt[safe], t_ref[safe])
    # planted divergence from the GPU's own self-consistent targets: accept == d
    announce("8b slice self-consistent candidates")
    g_tgt = V.self_consistent_candidates(model, t0, ctx, lay.block_table, nz, caches, K, first=toks_cand)
    d = wl.rng(46).integers(0, K + 1, size=R)
    cand = wl.plant_divergence(g_tgt, d, sh.vocab, 46)
    b2 = V.make_batch(t0, cand, ctx, lay.block_table, nz)
    announce("8b slice planted")
    _, tgt2, acc2, nxt2 = model.verify(b2, caches)
    sync()
    assert np.array_equal(acc2.cpu().numpy(), d)
    for r in range(R):
        assert nxt2.cpu().numpy()[r] == (g_tgt[r, d[r]] if d[r] < K else -1)
    # subset invariance: each request alone gives the same logits bits
    full = bits(model.verify(b2, caches)[0]).reshape(R, K, -1).copy()
    for r in [2, 0]:
        bb = V.make_batch(t0[[r]], cand[[r]], ctx[[r]], lay.block_table[[r]], nz[[r]])
        announce("8b slice alone", r)
        one = bits(model.verify(bb, caches)[0]).reshape(1, K, -1)
        assert np.array_equal(one[0], full[r])


def test_llama8b_slice_graph_replay_matches_eager(V):
    """The verifier step captured as one HIP graph replays to the eager step's
    bits: logits, targets and decisions, on three replays with other eager
    steps (another candidate batch over the same cache slots) and host
    synchronisations between them."""
    sh = wl.LLAMA3_8B
    R, K = 4, 8
    ctx = wl.context_lengths(52, R, 1500, 3000)
    announce("8b slice graph setup", list(ctx))
    _, _, model, lay, caches = _slice_world(V, ctx, seed=53)
    t0 = wl.tokens(54, (R,), sh.vocab)
    pos = ctx[:, None] + np.arange(K)[None, :] + 1
    nz = wl.gumbel_noise(56, np.repeat(np.arange(R), K).reshape(R, K), pos, sh.vocab)
    b = V.make_batch(t0, wl.tokens(55, (R, K), sh.vocab), ctx, lay.block_table, nz)
    other = V.make_batch(t0, wl.tokens(57, (R, K), sh.vocab), ctx, lay.block_table, nz)
    logits, tgt, acc, nxt = model.verify(b, caches)
    sync()
    ref = [bits(logits).copy(), tgt.cpu().numpy().copy(), acc.cpu().numpy().copy(), nxt.cpu().numpy().copy()]
    announce("8b slice graph capture")
    graph = model.capture(b, caches)
    for i in range(3):
        model.verify(other, caches)
        sync()
        announce("8b slice graph replay", i)
        for t in (b.target, b.accept_len, b.next_token):
            t.fill_(-7)
        sync()
        graph.replay()
        sync()
        got = [bits(model._buffers(R * K)["logits"]), b.target.cpu().numpy(), b.accept_len.cpu().numpy(),
               b.next_token.cpu().numpy()]
        for g_, r_, what in zip(got, ref, ["logits", "target", "accept_len", "next_token"]):
            assert np.array_equal(g_, r_), f"replay {i}: {what}"
    del graph
    # the fused lm_head + Gumbel verification gives the same decisions, eager
    # and replayed
    announce("8b slice fused head")
    _, ftgt, facc, fnxt = model.verify(b, caches, fused_head=True)
    sync()
    for g_, r_, what in zip([ftgt.cpu().numpy(), facc.cpu().numpy(), fnxt.cpu().numpy()], ref[1:],
                            ["target", "accept_len", "next_token"]):
        assert np.array_equal(g_, r_), f"fused head: {what}"
    fgraph = model.capture(b, caches, fused_head=True)
    for i in range(2):
        model.verify(other, caches)
        for t in (b.target, b.accept_len, b.next_token):
            t.fill_(-7)
        sync()
        fgraph.replay()
        sync()
        for g_, r_, what in zip([b.target.cpu().numpy(), b.accept_len.cpu().numpy(), b.next_token.cpu().numpy()],
                                ref[1:], ["target", "accept_len", "next_token"]):
            assert np.array_equal(g_, r_), f"fused head replay {i}: {what}"
    del fgraph


def test_llama8b_slice_repeated_replays_are_bitwise_identical(V):
    """Run-to-run determinism of the whole step: 100 replays of the captured
    2-layer step (logits, targets and decisions) are bit for bit the first
    replay's.  A race in a kernel (an LDS slot read before its copy landed, a
    partial folded before it was written) would show up as a replay that
    differs; the loop stops at the first one."""
    sh = wl.LLAMA3_8B
    R, K = 8, 8
    ctx = wl.context_lengths(62, R, 1000, 9000)
    announce("8b slice repeated replays setup", list(ctx))
    _, _, model, lay, caches = _slice_world(V, ctx, seed=63)
    t0 = wl.tokens(64, (R,), sh.vocab)
    pos = ctx[:, None] + np.arange(K)[None, :] + 1
    nz = wl.gumbel_noise(66, np.repeat(np.arange(R), K).reshape(R, K), pos, sh.vocab)
    b = V.make_batch(t0, wl.tokens(65, (R, K), sh.vocab), ctx, lay.block_table, nz)
    graph = model.capture(b, caches)
    logits = model._buffers(R * K)["logits"]
    graph.replay()
    sync()
    ref = [bits(logits).copy(), b.target.cpu().numpy().copy(), b.accept_len.cpu().numpy().copy(),
           b.next_token.cpu().numpy().copy()]
    announce("8b slice repeated replays: 100")
    for i in range(100):
        graph.replay()
        sync()
        got = [bits(logits), b.target.cpu().numpy(), b.accept_len.cpu().numpy(), b.next_token.cpu().numpy()]
        for g_, r_, what in zip(got, ref, ["logits", "target", "accept_len", "next_token"]):
            assert np.array_equal(g_, r_), f"replay {i + 1}: {what} differs from the first replay"
    del graph
