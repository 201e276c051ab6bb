"""Decode-verify-rollback around the batch-invariant verifier step.

LLM-42 post, paragraphs 3-4: a fast path decodes with the ordinary
(non-invariant) kernels; every K tokens, one batch-invariant verifier pass over
those K tokens of all N requests recomputes them at a fixed shape, overwrites
the fast path's KV with its own values, accepts the prefix whose tokens it
reproduces, and replaces the first token it does not reproduce with its own;
the fast path's later tokens are rolled back.  Reading-club post on Gumbel
coupling: both sides sample by Gumbel-max with the noise of the token's
(request, absolute position), so the fast path proposes exactly the verifier's
token wherever their logits agree closely enough, and the committed stream is
the stream the invariant kernels would produce one token at a time.

Here the fast path runs the same decoder with split-K GEMMs
(``gemm_splitk``) and load-adaptive attention splits
(``attn_decode_adaptive``), one token per request per forward.  Noise
comes from a caller-supplied function of (requests, positions), prepared in
advance like the verifier's.  Everything runs through the HIP library; the
host only moves the K sampled tokens and the accepted lengths.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

from . import _lib as L
from . import verifier as V


def _event_ms(fn, iters=5, warmup=2):
    for _ in range(warmup):
        fn()
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(iters):
        fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / iters


class SplitKernels:
    """The decoder's GEMMs and attention swapped for their non-invariant
    counterparts: split-K GEMMs (``gemm_splitk``) and attention whose KV split
    follows the load (``attn_decode_adaptive``).  Owns its workspaces; pass
    ``gemm_fn=sk.gemm, attn_fn=sk.attn`` to ``VerifierModel.forward``.

    tune=False: the library's automatic choices (splits from the staged
    kernel's own grid; the attention split from the batch).  tune=True: the
    first call of each shape times the candidates -- 1, 2, 4 and 8 splits
    (1 is the invariant kernel itself), KV splits of 256 * 2^k tokens up to
    the longest context -- into scratch outputs and keeps the fastest, as a
    serving engine tuned for speed rather than invariance would.  The tuning
    runs eagerly (never inside a graph capture)."""

    GEMM_SPLITS = (1, 2, 4, 8)

    def __init__(self, R, Hkv, max_blocks, device="cuda", tune=False):
        self.device, self.tune = device, tune
        self.max_blocks = max_blocks
        self.split = L.attn_adaptive_split(R, Hkv, max_blocks)
        self.attn_splits = {}
        self.attn_ws = torch.empty(max(L.attn_workspace_bytes(R, Hkv, max_blocks, 256 if tune else self.split), 16),
                                   dtype=torch.uint8, device=device)
        self.gemm_ws = {}
        self.splits = {}
        self.timings = {}

    def _ws(self, M, N, sp):
        ws = self.gemm_ws.get((M, N, sp))
        if ws is None:
            ws = torch.empty(max(L.splitk_workspace_bytes(M, N, sp), 16), dtype=torch.uint8, device=self.device)
            self.gemm_ws[(M, N, sp)] = ws
        return ws

    def _choose_splits(self, a, b, c, accumulate, swiglu):
        M, K = a.shape
        N = b.shape[0]
        key = (M, N, K)
        if key not in self.splits:
            if not self.tune:
                self.splits[key] = L.splitk_auto_splits(M, N, K)
            else:
                scratch = torch.zeros_like(c)
                t = {sp: _event_ms(lambda sp=sp: L.gemm_splitk(a, b, scratch, sp, self._ws(M, N, sp),
                                                               accumulate=accumulate, swiglu=swiglu))
                     for sp in self.GEMM_SPLITS if K % (64 * sp) == 0}
                self.timings[("gemm", M, N, K)] = {sp: round(ms * 1e3, 2) for sp, ms in t.items()}
                self.splits[key] = min(t, key=t.get)
        return self.splits[key]

    def gemm(self, a, b, c, accumulate=False, swiglu=False):
        M, K = a.shape
        N = b.shape[0]
        sp = self._choose_splits(a, b, c, accumulate, swiglu)
        return L.gemm_splitk(a, b, c, sp, self._ws(M, N, sp), accumulate=accumulate, swiglu=swiglu)

    def attn(self, q, k_cache, v_cache, block_table, ctx, out, q_len, scale, workspace=None):
        split = self.split
        if self.tune:
            key = (block_table.shape[0], q_len)
            if key not in self.attn_splits:
                scratch = torch.empty_like(out)
                cands, sp = [], 256
                while True:
                    cands.append(sp)
                    if sp >= self.max_blocks * 16:
                        break
                    sp *= 2
                t = {sp: _event_ms(lambda sp=sp: L.attn_decode_adaptive(q, k_cache, v_cache, block_table, ctx,
                                                                        scratch, q_len, scale, self.attn_ws,
                                                                        split_tokens=sp))
                     for sp in cands}
                self.timings[("attn",) + key] = {sp: round(ms * 1e3, 2) for sp, ms in t.items()}
                self.attn_splits[key] = min(t, key=t.get)
            split = self.attn_splits[key]
        return L.attn_decode_adaptive(q, k_cache, v_cache, block_table, ctx, out, q_len, scale, self.attn_ws,
                                      split_tokens=split)


@dataclass
class RoundStats:
    """Per-round bookkeeping of a decode-verify-rollback run."""

    accept_len: list = field(default_factory=list)  # [rounds] arrays [R]: verifier-accepted draft prefix
    committed: list = field(default_factory=list)  # [rounds] arrays [R]: tokens committed (prefix + fix)

    def acceptance(self, K):
        """Fraction of drafted tokens the verifier accepted."""
        a = np.concatenate(self.accept_len) if self.accept_len else np.zeros(0)
        return float(a.mean() / K) if a.size else float("nan")

    def tokens_per_round(self):
        """Mean tokens committed per request per round (E[L] of the pages)."""
        c = np.concatenate(self.committed) if self.committed else np.zeros(0)
        return float(c.mean()) if c.size else float("nan")


class DecodeVerifyRollback:
    """Decode-verify-rollback for R requests on a bf16 ``VerifierModel``.

    ``block_table`` [R, max_blocks] (host int32) must cover every position the
    run reaches; ``noise_fn(requests, positions)`` returns the fp32 Gumbel rows
    [n, vocab] (device) of those (request, absolute position) keys.
    ``fast`` chooses the draft kernels: "split" (split-K + adaptive attention
    splits) or "invariant" (the verifier's own kernels, which must then be
    accepted in full).
    """

    def __init__(self, model: V.VerifierModel, caches, block_table, K, noise_fn, fast="split", device="cuda"):
        self.model, self.caches, self.K, self.noise_fn, self.device = model, caches, K, noise_fn, device
        self.bt_host = np.ascontiguousarray(block_table, dtype=np.int32)
        self.bt = torch.from_numpy(self.bt_host).to(device)
        R, mb = self.bt_host.shape
        self.R = R
        self.req = np.arange(R)
        if fast == "split":
            self.kern = SplitKernels(R, model.shape.kv_heads, mb, device)
            self.fast_kw = dict(gemm_fn=self.kern.gemm, attn_fn=self.kern.attn)
        elif fast == "invariant":
            self.kern = None
            self.fast_kw = {}
        else:
            raise ValueError(f"fast must be 'split' or 'invariant', not {fast!r}")
        self._cand0 = torch.zeros((R, 1), dtype=torch.int32, device=device)
        self._tgt = torch.empty((R, 1), dtype=torch.int32, device=device)
        self._acc = torch.empty(R, dtype=torch.int32, device=device)
        self._nxt = torch.empty(R, dtype=torch.int32, device=device)
        self.stats = RoundStats()

    def _slots(self, pos):
        page = self.bt_host[self.req, pos // 16]
        if (page < 0).any():
            raise ValueError("block table does not cover the positions being decoded")
        return page.astype(np.int64) * 16 + pos % 16

    def _dev(self, a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(self.device)

    def decode_one(self, tok, pos, **kernels):
        """One token per request: the token ``tok`` [R] (host array or device
        int32 tensor) at absolute position ``pos`` [R] (its K/V written to that
        position's slot; it attends to positions 0 .. pos), then the
        Gumbel-max sample of position pos + 1.  Returns the sampled tokens as
        a device int32 tensor [R], valid until the next call."""
        if not isinstance(tok, torch.Tensor):
            tok = self._dev(np.asarray(tok, np.int32))
        pos = np.asarray(pos, np.int32)
        pos_d = self._dev(pos)
        logits = self.model.forward(tok, pos_d, pos_d, 1, self.bt, self._dev(self._slots(pos)), self.caches,
                                    **kernels)
        noise = self.noise_fn(self.req, pos + 1)
        L.gumbel_verify(logits, noise, self._cand0, self._tgt, self._acc, self._nxt)
        return self._tgt.view(-1)

    def draft(self, t0, ctx):
        """K tokens per request from the fast path, starting after t0 at
        position ctx.  Returns host int32 [R, K]."""
        out = torch.empty((self.R, self.K), dtype=torch.int32, device=self.device)
        tok = np.asarray(t0, np.int32)
        ctx = np.asarray(ctx, np.int32)
        for j in range(self.K):
            out[:, j] = self.decode_one(tok, ctx + j, **self.fast_kw)
            tok = out[:, j].contiguous()  # the next forward's input, kept on the device
        return out.cpu().numpy()

    def verify(self, t0, cand, ctx):
        """The batch-invariant verifier step over the drafted tokens; returns
        (accept_len, next_token) on the host."""
        ctx = np.asarray(ctx, np.int32)
        pos = ctx[:, None] + np.arange(self.K, dtype=np.int32)[None, :] + 1
        noise = self.noise_fn(np.repeat(self.req, self.K), pos.reshape(-1))
        batch = V.make_batch(t0, cand, ctx, self.bt_host, noise, device=self.device)
        _, _, acc, nxt = self.model.verify(batch, self.caches)
        return acc.cpu().numpy(), nxt.cpu().numpy()

    def round(self, t0, ctx, draft_fn=None):
        """Draft K tokens (fast path, or ``draft_fn(t0, ctx)`` [R, K]), verify,
        roll back.  Returns (new ctx, committed token lists, new t0)."""
        cand = self.draft(t0, ctx) if draft_fn is None else np.asarray(draft_fn(t0, ctx), np.int32)
        acc, nxt = self.verify(t0, cand, ctx)
        new_ctx, committed, new_t0 = V.rollback(ctx, acc, nxt, cand)
        self.stats.accept_len.append(acc.copy())
        self.stats.committed.append(np.asarray([len(c) for c in committed]))
        return new_ctx, committed, new_t0

    def run(self, t0, ctx, rounds, draft_fn=None):
        """Exactly ``rounds`` rounds; returns each request's committed tokens
        (a list of R lists; every round commits between 1 and K per request,
        so positions up to ctx + rounds*K - 1 must be covered)."""
        hist = [[] for _ in range(self.R)]
        t0 = np.asarray(t0, np.int32)
        ctx = np.asarray(ctx, np.int32)
        for _ in range(rounds):
            ctx, committed, t0 = self.round(t0, ctx, draft_fn)
            for r in range(self.R):
                hist[r].extend(committed[r])
        return hist

    def decode(self, t0, ctx, n_tokens, draft_fn=None):
        """Run rounds until every request has at least n_tokens committed;
        returns host int32 [R, n_tokens] (the first n of each stream).  Requests
        ahead of the slowest keep decoding, so the block table must cover the
        positions they reach."""
        hist = [[] for _ in range(self.R)]
        t0 = np.asarray(t0, np.int32)
        ctx = np.asarray(ctx, np.int32)
        while min(len(h) for h in hist) < n_tokens:
            ctx, committed, t0 = self.round(t0, ctx, draft_fn)
            for r in range(self.R):
                hist[r].extend(committed[r])
        return np.asarray([h[:n_tokens] for h in hist], np.int32)

    def sequential(self, t0, ctx, n_tokens, **kernels):
        """One token per forward for n_tokens steps (the invariant kernels by
        default; the fast path's with ``**self.fast_kw``).  Returns host int32
        [R, n_tokens]: the stream decode-verify-rollback must reproduce when
        the kernels are the invariant ones."""
        out = torch.empty((self.R, n_tokens), dtype=torch.int32, device=self.device)
        tok = np.asarray(t0, np.int32)
        ctx = np.asarray(ctx, np.int32)
        for j in range(n_tokens):
            out[:, j] = self.decode_one(tok, ctx + j, **kernels)
            tok = out[:, j].contiguous()
        return out.cpu().numpy()

