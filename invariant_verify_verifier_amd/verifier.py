"""The verifier step: decoder forward over W = N*K candidate tokens, Gumbel-max
verification and the rollback rule.

LLM-42 post, paragraph 3: the fast path decodes with ordinary kernels and
produces candidate tokens; the verifier -- a forward at a fixed batch, the
ground truth -- checks them, starting from the last token known to be
correct, and at every verification overwrites the fast path's KV with its own
values.  Paragraph 4: the verifier takes K tokens from each of N requests, so
W = N*K is both its batch and the number of tokens it checks.  The reading-club
post on Gumbel coupling gives the check itself: with the noise shared between
draft and target, accept while the tokens agree.

This module only sequences library calls and owns device buffers; every
arithmetic step runs in libbiverify's kernels.  Inputs for request r are
[t0_r, c_0, .., c_{K-2}] at positions L_r .. L_r+K-1; output j predicts
position L_r + j + 1 and is compared with c_j.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np
import torch

from . import _lib as L


@dataclass
class Shape:
    layers: int
    hidden: int
    heads: int
    kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    eps: float = 1e-6
    rope_theta: float = 500000.0

    @property
    def q_cols(self):
        return self.heads * self.head_dim

    @property
    def kv_cols(self):
        return self.kv_heads * self.head_dim

    @property
    def qkv_cols(self):
        return self.q_cols + 2 * self.kv_cols


def _t(a, dtype, device):
    """numpy input (fp32 values or bf16 bit patterns) -> device tensor."""
    a = np.ascontiguousarray(a)
    if dtype == torch.bfloat16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a.astype(np.float32)).to(device)


class VerifierModel:
    """Decoder weights on the GPU and the verifier forward.

    Weight layout [out_features, in_features]; Q, K, V projections fused into
    one [Hq*D + 2*Hkv*D, H] matrix and gate/up into one [2F, H] matrix, so one
    GEMM produces each (gate/up interleaved in 32-row blocks, so that the bf16
    GEMM applies SwiGLU in its epilogue).  The residual stream is fp32; GEMM
    inputs are the model dtype (bf16: MFMA; fp32: FMA path).
    """

    def __init__(self, shape: Shape, dtype: torch.dtype, layers, embed, lm_head, final_norm, max_pos=65536,
                 device="cuda"):
        self.shape, self.dtype, self.device = shape, dtype, device
        # the model's own layer dicts: gate/up weights repacked once into the
        # interleaved layout of the SwiGLU epilogue (the caller's tensors are
        # left as they are)
        self.layers = [dict(lw, w_gu=L.pack_gate_up(lw["w_gu"])) for lw in layers]
        self.embed, self.lm_head, self.final_norm = embed, lm_head, final_norm
        self.max_pos = max_pos
        self.rope = L.rope_table(max_pos, shape.head_dim, shape.rope_theta).to(device)
        self._bufs = {}
        self._ws = {}
        self._gumbel_ws = {}

    # ------------------------------------------------------------ construction

    @classmethod
    def from_host(cls, w, device="cuda", max_pos=65536):
        """From workloads.ModelWeights (numpy; fp32 values or bf16 bits)."""
        s = w.shape
        shape = Shape(s.layers if not w.layers else len(w.layers), s.hidden, s.heads, s.kv_heads, s.head_dim, s.ffn,
                      s.vocab, s.eps, s.rope_theta)
        dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        layers = []
        for lw in w.layers:
            layers.append(dict(
                attn_norm=_t(lw["attn_norm"], dt, device),
                wqkv=_t(np.concatenate([lw["wq"], lw["wk"], lw["wv"]], axis=0), dt, device),
                wo=_t(lw["wo"], dt, device),
                ffn_norm=_t(lw["ffn_norm"], dt, device),
                w_gu=_t(np.concatenate([lw["w_gate"], lw["w_up"]], axis=0), dt, device),
                w_down=_t(lw["w_down"], dt, device),
            ))
        return cls(shape, dt, layers, _t(w.embed, dt, device), _t(w.lm_head, dt, device),
                   _t(w.final_norm, dt, device), max_pos=max_pos, device=device)

    def alloc_kv(self, num_blocks, fill=None):
        sh = self.shape
        caches = []
        for _ in range(sh.layers):
            k = torch.zeros((num_blocks, sh.kv_heads, 16, sh.head_dim), dtype=self.dtype, device=self.device)
            v = torch.zeros_like(k)
            caches.append((k, v))
        return caches

    # ------------------------------------------------------------ buffers

    def _buffers(self, W):
        b = self._bufs.get(W)
        if b is None:
            sh, dt, dev = self.shape, self.dtype, self.device
            b = dict(
                x=torch.empty((W, sh.hidden), dtype=torch.float32, device=dev),
                h=torch.empty((W, sh.hidden), dtype=dt, device=dev),
                qkv=torch.empty((W, sh.qkv_cols), dtype=dt, device=dev),
                attn=torch.empty((W, sh.heads, sh.head_dim), dtype=dt, device=dev),
                gu=torch.empty((W, 2 * sh.ffn), dtype=dt, device=dev),
                act=torch.empty((W, sh.ffn), dtype=dt, device=dev),
                logits=torch.empty((W, sh.vocab), dtype=torch.float32, device=dev),
            )
            self._bufs[W] = b
        return b

    def workspace(self, R, max_blocks, q_len=1):
        key = (R, max_blocks, q_len)
        ws = self._ws.get(key)
        if ws is None:
            nbytes = L.attn_workspace_bytes(R, self.shape.kv_heads, max_blocks, q_len=q_len, Hq=self.shape.heads)
            ws = torch.zeros(max(nbytes, 16), dtype=torch.uint8, device=self.device)
            self._ws[key] = ws
        return ws

    # ------------------------------------------------------------ forward

    def forward(self, tokens, pos, ctx, q_len, block_table, slots, caches, attn_fn=None, gemm_fn=None, head=True):
        """tokens/pos [W] int32, ctx [R] int32, block_table [R, mb] int32, slots [W] int64 (device).
        Returns fp32 logits [W, V] (a buffer reused by the next call with the same W), or with
        head=False the final-normed hidden rows [W, H] that the lm_head would multiply."""
        sh = self.shape
        W = tokens.shape[0]
        R, mb = block_table.shape
        b = self._buffers(W)
        x, h, qkv, attn, gu, act, logits = b["x"], b["h"], b["qkv"], b["attn"], b["gu"], b["act"], b["logits"]
        ws = self.workspace(R, mb, q_len) if self.dtype == torch.bfloat16 else None
        scale = 1.0 / math.sqrt(sh.head_dim)
        gemm = gemm_fn or L.gemm_bi
        attend = attn_fn or L.attn_decode_bi
        qc = sh.q_cols
        L.embed_rows(tokens, self.embed, x)
        for li, lw in enumerate(self.layers):
            k_cache, v_cache = caches[li]
            L.rmsnorm_bi(x, lw["attn_norm"], h, sh.eps)
            gemm(h, lw["wqkv"], qkv)
            L.rope_kv_overwrite(qkv, pos, self.rope, slots, k_cache, v_cache, sh.heads)
            attend(qkv[:, :qc], k_cache, v_cache, block_table, ctx, attn, q_len, scale, ws)
            gemm(attn.view(W, qc), lw["wo"], x, accumulate=True)
            L.rmsnorm_bi(x, lw["ffn_norm"], h, sh.eps)
            if self.dtype == torch.bfloat16:  # SwiGLU in the matmul's epilogue
                gemm(h, lw["w_gu"], act, swiglu=True)
            else:
                gemm(h, lw["w_gu"], gu)
                L.swiglu(gu, act, block=L.SWIGLU_BLOCK)
            gemm(act, lw["w_down"], x, accumulate=True)
        L.rmsnorm_bi(x, self.final_norm, h, sh.eps)
        if not head:
            return h
        gemm(h, self.lm_head, logits)
        return logits

    def capture(self, step, caches, **kw):
        """Record one verifier step (forward + Gumbel verify) as a HIP graph.

        The step's ~200 kernel launches then replay with no host work and no
        launch gaps between them.  A replay reads the inputs from, and writes
        the outputs to, the tensors of ``step``, the model's buffers and the
        caches, so new data is written into those tensors in place before
        ``graph.replay()``.  One eager step runs first so that every buffer and
        workspace exists before the capture: the graph then holds kernel nodes
        only (no kernel of the step allocates memory or clears it through the
        runtime)."""
        self.verify(step, caches, **kw)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            self.verify(step, caches, **kw)
        return graph

    def verify(self, step, caches, fused_head=False, **kw):
        """One verifier step.  `step` is a VerifyBatch already on the device.
        Returns (logits [W,V], target [R,K], accept_len [R], next_token [R]).
        fused_head=True (bf16 model): the lm_head matmul and the Gumbel
        verification run as one call that never stores the logits (the same
        decisions as the invariant lm_head + gumbel_verify, bit for bit);
        logits is then None.  The fused lm_head is the invariant one whatever
        ``gemm_fn`` the layers use."""
        if fused_head:
            if self.dtype != torch.bfloat16:
                raise ValueError("fused_head needs the bf16 model")
            h = self.forward(step.tokens, step.pos, step.ctx, step.K, step.block_table, step.slots, caches,
                             head=False, **kw)
            W = h.shape[0]
            ws = self._gumbel_ws.get(W)
            if ws is None:
                ws = torch.empty(L.gumbel_workspace_bytes(W, self.shape.vocab), dtype=torch.uint8,
                                 device=self.device)
                self._gumbel_ws[W] = ws
            L.lm_head_gumbel_verify(h, self.lm_head, step.noise, step.cand, step.target, step.accept_len,
                                    step.next_token, ws)
            return None, step.target, step.accept_len, step.next_token
        logits = self.forward(step.tokens, step.pos, step.ctx, step.K, step.block_table, step.slots, caches, **kw)
        L.gumbel_verify(logits, step.noise, step.cand, step.target, step.accept_len, step.next_token)
        return logits, step.target, step.accept_len, step.next_token


@dataclass
class VerifyBatch:
    """Device inputs/outputs of one verifier step for R requests x K candidates."""

    K: int
    tokens: torch.Tensor  # [R*K] int32: t0, c_0 .. c_{K-2}
    pos: torch.Tensor  # [R*K] int32: L_r + j
    ctx: torch.Tensor  # [R] int32: L_r
    block_table: torch.Tensor  # [R, max_blocks] int32
    slots: torch.Tensor  # [R*K] int64: physical slot of position L_r + j
    cand: torch.Tensor  # [R, K] int32
    noise: torch.Tensor  # [R*K, V] fp32: noise of position L_r + j + 1
    target: torch.Tensor
    accept_len: torch.Tensor
    next_token: torch.Tensor


def make_batch(t0, cand, ctx, block_table, noise, device="cuda") -> VerifyBatch:
    """Host-side scheduler bookkeeping for one verifier step: token rows,
    positions and cache slots from the block tables (numpy in, device out)."""
    t0 = np.asarray(t0, dtype=np.int32)
    cand = np.asarray(cand, dtype=np.int32)
    ctx = np.asarray(ctx, dtype=np.int32)
    bt = np.asarray(block_table, dtype=np.int32)
    R, K = cand.shape
    toks = np.concatenate([t0[:, None], cand[:, :K - 1]], axis=1).reshape(-1)
    pos = (ctx[:, None] + np.arange(K, dtype=np.int32)[None, :]).reshape(-1)
    rows = np.repeat(np.arange(R), K)
    slots = bt[rows, pos // 16].astype(np.int64) * 16 + pos % 16
    if (bt[rows, pos // 16] < 0).any():
        raise ValueError("block table does not cover positions L_r .. L_r+K-1")
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)
    nz = noise if isinstance(noise, torch.Tensor) else torch.from_numpy(np.ascontiguousarray(noise, dtype=np.float32))
    return VerifyBatch(
        K=K, tokens=dev(toks), pos=dev(pos), ctx=dev(ctx), block_table=dev(bt), slots=dev(slots), cand=dev(cand),
        noise=nz.reshape(R * K, -1).to(device), target=torch.empty((R, K), dtype=torch.int32, device=device),
        accept_len=torch.empty(R, dtype=torch.int32, device=device),
        next_token=torch.empty(R, dtype=torch.int32, device=device))


@dataclass
class TreeBatch:
    """A verifier step over B chains per request (tree verification by
    branches): ``chains`` is the VerifyBatch of the R*B chains, chain b of
    request r at row block r*B + b; the page copies give every chain after the
    first a private copy of the page holding position L_r (and private pages
    for the rest of L_r .. L_r+K-1)."""

    R: int
    B: int
    chains: VerifyBatch
    copy_src: torch.Tensor  # [n] int32 pages copied into ...
    copy_dst: torch.Tensor  # [n] int32 ... the chains' private pages
    best: torch.Tensor  # [R] int32 outputs of tree_select
    accept_len: torch.Tensor
    next_token: torch.Tensor


def make_tree_batch(t0, chains, ctx, block_table, private_pages, noise, device="cuda") -> TreeBatch:
    """Host bookkeeping for tree verification by branches.

    chains [R, B, K] int32: the candidate tokens of each root-to-leaf chain of
    request r's draft tree (chains may share prefixes).  block_table [R, mb]:
    the requests' tables, covering positions up to L_r + K - 1 (chain 0 uses
    them as they are).  private_pages [R, B-1, P] int32: for chains 1..B-1,
    the P = ceil((L_r % 16 + K) / 16) pages that replace the request's pages
    from page L_r // 16 on; the first of them receives a copy of the request's
    page L_r // 16 (its context tokens).  noise [R, K, V]: the noise row of
    the position each output samples, shared by all chains of a request (the
    key is the request and the absolute position)."""
    chains = np.asarray(chains, dtype=np.int32)
    R, B, K = chains.shape
    ctx = np.asarray(ctx, dtype=np.int32)
    bt = np.asarray(block_table, dtype=np.int32)
    priv = np.asarray(private_pages, dtype=np.int32).reshape(R, B - 1, -1) if B > 1 else None
    rows_bt = np.repeat(bt, B, axis=0).copy()  # [R*B, mb]
    src, dst = [], []
    for r in range(R):
        p0 = int(ctx[r]) // 16
        n_pages = (int(ctx[r]) % 16 + K + 15) // 16
        for b in range(1, B):
            pages = priv[r, b - 1, :n_pages]
            rows_bt[r * B + b, p0:p0 + n_pages] = pages
            src.append(int(bt[r, p0]))
            dst.append(int(pages[0]))
    t0s = np.repeat(np.asarray(t0, dtype=np.int32), B)
    nz = noise if isinstance(noise, torch.Tensor) else torch.from_numpy(np.ascontiguousarray(noise, dtype=np.float32))
    nz = nz.reshape(R, 1, K, -1).expand(R, B, K, nz.shape[-1]).reshape(R * B * K, -1).contiguous()
    cb = make_batch(t0s, chains.reshape(R * B, K), np.repeat(ctx, B), rows_bt, nz, device=device)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.int32))).to(device)
    return TreeBatch(R=R, B=B, chains=cb, copy_src=dev(src), copy_dst=dev(dst),
                     best=torch.empty(R, dtype=torch.int32, device=device),
                     accept_len=torch.empty(R, dtype=torch.int32, device=device),
                     next_token=torch.empty(R, dtype=torch.int32, device=device))


def verify_tree(model, tb: TreeBatch, caches, **kw):
    """One verifier step over every chain of every request's draft tree: copy
    the context page into the chains' private pages (every layer), run the
    ordinary verifier step over the R*B chains, then pick each request's chain
    with the longest accepted prefix.  Returns (best [R], accept_len [R],
    next_token [R], per-chain targets [R*B, K])."""
    if tb.copy_src.numel():
        for k_cache, v_cache in caches:
            L.kv_copy_pages(tb.copy_src, tb.copy_dst, k_cache, v_cache)
    _, target, acc, nxt = model.verify(tb.chains, caches, **kw)
    L.tree_select(acc.view(tb.R, tb.B), nxt.view(tb.R, tb.B), tb.best, tb.accept_len, tb.next_token)
    return tb.best, tb.accept_len, tb.next_token, target


def adopt_chain_pages(block_table, ctx, best, private_pages, K):
    """Host bookkeeping after tree verification: request r keeps the pages of
    its selected chain best[r] for positions L_r .. L_r+K-1 (chain 0 uses the
    request's own pages; chain b >= 1 its private ones, whose first page
    already holds a copy of the request's context tokens).  Returns the new
    block table [R, mb] and, per request, the pages no longer in use (the
    request's replaced pages and the other chains' private pages)."""
    bt = np.array(block_table, dtype=np.int32, copy=True)
    ctx = np.asarray(ctx)
    best = np.asarray(best)
    R = bt.shape[0]
    priv = None if private_pages is None else np.asarray(private_pages, dtype=np.int32)
    freed = []
    for r in range(R):
        p0 = int(ctx[r]) // 16
        n_pages = (int(ctx[r]) % 16 + K + 15) // 16
        b = int(best[r])
        mine = [] if priv is None else [int(x) for x in priv[r].reshape(priv.shape[1], -1)[:, :n_pages].ravel()]
        if b > 0:
            chosen = [int(x) for x in priv[r, b - 1, :n_pages]]
            out = [int(x) for x in bt[r, p0:p0 + n_pages]] + [x for x in mine if x not in chosen]
            bt[r, p0:p0 + n_pages] = chosen
        else:
            out = mine
        freed.append(out)
    return bt, freed


def self_consistent_candidates(model, t0, ctx, block_table, noise, caches, K, first=None, **kw):
    """Candidates that equal the verifier's own targets at every position.

    Target j depends on the inputs at positions <= j, i.e. on candidates
    0 .. j-1, so feeding the targets back as candidates fixes at least one
    more position per pass; K passes reach the fixed point.  Used to plant a
    first divergence at a chosen position (accept_len must then equal it).
    """
    R = len(t0)
    cand = np.zeros((R, K), np.int32) if first is None else np.asarray(first, np.int32)
    for _ in range(K):
        b = make_batch(t0, cand, ctx, block_table, noise)
        _, tgt, _, _ = model.verify(b, caches, **kw)
        new = tgt.cpu().numpy()
        if np.array_equal(new, cand):
            break
        cand = new
    return cand


def rollback(ctx, accept_len, next_token, cand):
    """Host rule after a verification: keep the accepted prefix, take the
    verifier's token at the first divergence, and continue from there.
    Returns (new ctx, committed tokens per request, new reference token)."""
    ctx = np.asarray(ctx)
    a = np.asarray(accept_len)
    nx = np.asarray(next_token)
    cand = np.asarray(cand)
    K = cand.shape[1]
    out_ctx = ctx + np.minimum(a + 1, K)
    committed, t0 = [], []
    for r in range(len(ctx)):
        toks = list(cand[r, :a[r]]) + ([int(nx[r])] if a[r] < K else [])
        committed.append([int(t) for t in toks])
        t0.append(int(toks[-1]))
    return out_ctx.astype(np.int32), committed, np.asarray(t0, dtype=np.int32)
