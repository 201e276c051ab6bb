"""Decode-verify-rollback around the verifier step, on the Llama-3-8B-shaped
slice (2 of the 32 layers, bf16, 8 requests, contexts U[600, 4000], K = 8).

LLM-42 post, paragraphs 3-4, and the Gumbel-coupling post: whatever the fast
path drafts, the committed stream is the one that one-token-at-a-time decoding
with the batch-invariant kernels produces, bit for bit (the verifier's row j
sees the same inputs as that decode's step j and the same noise key).  Checked
for three fast paths: split-K GEMMs with load-adaptive attention splits (the
non-invariant kernels), a drafter with one planted wrong token per round, and
the invariant kernels themselves, whose drafts the verifier must accept in
full.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from gpu_util import DEV, announce

pytestmark = pytest.mark.gpu

R, K, ROUNDS, LAYERS = 8, 8, 3, 2
N_TOK = 2 * K  # tokens compared per request


@pytest.fixture(scope="module")
def world():
    import invariant_verify_verifier_amd.dvr as D
    import invariant_verify_verifier_amd.verifier as V

    assert torch.cuda.is_available()
    sh = wl.LLAMA3_8B
    ctx = wl.context_lengths(47, R, 600, 4000)
    announce("dvr slice setup", list(ctx))
    dw = wl.device_model_weights(sh, 40, layers=LAYERS)
    shape = V.Shape(LAYERS, sh.hidden, sh.heads, sh.kv_heads, sh.head_dim, sh.ffn, sh.vocab, sh.eps, sh.rope_theta)
    model = V.VerifierModel(shape, torch.bfloat16, dw["layers"], dw["embed"], dw["lm_head"], dw["final_norm"],
                            max_pos=8192)
    lay = wl.paged_layout(ctx, K * (ROUNDS + 3), seed=48)
    caches = wl.device_kv_cache(sh, lay.num_blocks, 41, layers=LAYERS)

    def noise_fn(req, pos):
        return torch.from_numpy(wl.gumbel_noise(49, req, pos, sh.vocab)).to(DEV)

    t0 = wl.tokens(50, (R,), sh.vocab)
    inv = D.DecodeVerifyRollback(model, caches, lay.block_table, K, noise_fn, fast="invariant")
    announce("dvr slice sequential invariant decode")
    seq = inv.sequential(t0, ctx, N_TOK + 2 * K)
    return dict(D=D, model=model, caches=caches, lay=lay, ctx=ctx, t0=t0, noise_fn=noise_fn, seq=seq, sh=sh)


def test_dvr_with_split_fast_path_reproduces_invariant_decode(world):
    w = world
    dvr = w["D"].DecodeVerifyRollback(w["model"], w["caches"], w["lay"].block_table, K, w["noise_fn"], fast="split")
    announce("dvr slice split-K fast path")
    out = dvr.decode(w["t0"], w["ctx"], N_TOK)
    st = dvr.stats
    print(f"dvr split fast path: acceptance {st.acceptance(K):.3f}, tokens per round {st.tokens_per_round():.2f}, "
          f"rounds {len(st.accept_len)}")
    assert np.array_equal(out, w["seq"][:, :N_TOK])
    # the fast path decoding on its own (no verification) for comparison: its
    # stream may leave the invariant one at a near-tie; report where
    announce("dvr slice split-K sequential decode")
    fast_seq = dvr.sequential(w["t0"], w["ctx"], N_TOK, **dvr.fast_kw)
    diff = np.argmax(fast_seq != w["seq"][:, :N_TOK], axis=1)
    same = (fast_seq == w["seq"][:, :N_TOK]).all(axis=1)
    print(f"split-K decode alone: {int(same.sum())} of {R} streams equal the invariant one; first differences at "
          f"{[int(d) for d, s in zip(diff, same) if not s]}")


def test_dvr_with_planted_wrong_drafts_rolls_back_exactly(world):
    w = world
    seq, ctx0 = w["seq"], w["ctx"]
    dvr = w["D"].DecodeVerifyRollback(w["model"], w["caches"], w["lay"].block_table, K, w["noise_fn"],
                                      fast="invariant")
    g = wl.rng(51)
    planted = []

    def drafter(t0, ctx):
        done = np.asarray(ctx) - ctx0  # tokens committed so far per request
        d = g.integers(0, K + 1, size=R)  # K: no wrong token this round
        cand = np.stack([seq[r, done[r]:done[r] + K] for r in range(R)]).astype(np.int32)
        for r in range(R):
            if d[r] < K:
                cand[r, d[r]] = (cand[r, d[r]] + 1 + g.integers(0, w["sh"].vocab - 1)) % w["sh"].vocab
        planted.append(d)
        return cand

    announce("dvr slice planted drafts")
    hist = dvr.run(w["t0"], ctx0, ROUNDS, draft_fn=drafter)
    for r in range(R):
        assert np.array_equal(np.asarray(hist[r], np.int32), seq[r, :len(hist[r])]), r
    for d, a in zip(planted, dvr.stats.accept_len):
        assert np.array_equal(a, d), (d, a)
    assert sum(len(h) for h in hist) < R * ROUNDS * K  # some drafts were rolled back


def test_dvr_with_invariant_fast_path_accepts_every_draft(world):
    w = world
    dvr = w["D"].DecodeVerifyRollback(w["model"], w["caches"], w["lay"].block_table, K, w["noise_fn"],
                                      fast="invariant")
    announce("dvr slice invariant fast path")
    out = dvr.decode(w["t0"], w["ctx"], N_TOK)
    assert np.array_equal(out, w["seq"][:, :N_TOK])
    assert dvr.stats.acceptance(K) == 1.0
    assert dvr.stats.tokens_per_round() == K
