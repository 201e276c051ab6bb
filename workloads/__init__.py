"""Seeded synthetic inputs for the batch-invariant verifier step.

This module is shared by the HIP path's tests/bench and by the CPU oracle's
tests.  It only *makes inputs*: random tensors, bf16 bit patterns, paged-cache
layouts, candidate vectors and the Gumbel noise table.  It holds none of the
verifier's arithmetic (no norm, no product, no softmax, no argmax, no verify
rule), so that the oracle and the kernels can be compared on identical bits.

The noise table is an input because the method draws its random numbers before
the forward pass runs (the reading-club post on Gumbel coupling, "Gumbel-Max
trick" paragraph: the noise does not depend on the logits and can be prepared
in advance).  It is generated here from a counter-based hash keyed by
(seed, request, absolute position of the sampled token, vocab id), so the draft
and target sides of a coupled decode see the same noise for the same position.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

# ---------------------------------------------------------------------------
# bf16 bit patterns (inputs are handed to both sides as identical bits)
# ---------------------------------------------------------------------------


def bf16_bits(x) -> np.ndarray:
    """fp32 values -> bf16 bit patterns (uint16), round to nearest even.

    NaN stays NaN (quiet); infinities stay infinite.
    """
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    rounded = ((u + 0x7FFF + lsb) >> 16).astype(np.uint32)
    nan = np.isnan(f)
    rounded = np.where(nan, ((u >> 16) | 0x40).astype(np.uint32), rounded)
    return rounded.astype(np.uint16)


def bf16_to_f32(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> fp32 values (exact)."""
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (b.astype(np.uint32) << 16).view(np.float32)


def rng(seed, *stream) -> np.random.Generator:
    """Independent NumPy generator for (seed, stream...)."""
    return np.random.default_rng([int(seed), *[int(s) for s in stream]])


def normal_f32(seed, shape, std=1.0, mean=0.0, stream=()) -> np.ndarray:
    """N(mean, std^2) drawn in fp64 and rounded once to fp32."""
    g = rng(seed, *stream)
    return (g.standard_normal(size=shape) * std + mean).astype(np.float32)


def normal_bf16(seed, shape, std=1.0, mean=0.0, stream=()) -> np.ndarray:
    """N(mean, std^2) drawn in fp64 -> fp32 -> bf16 (RNE); returns uint16 bits."""
    return bf16_bits(normal_f32(seed, shape, std, mean, stream))


# ---------------------------------------------------------------------------
# Counter-based Gumbel noise table
# ---------------------------------------------------------------------------

_PHI = np.uint64(0x9E3779B97F4A7C15)  # splitmix64 increment (golden ratio)
_C1 = np.uint64(0xBF58476D1CE4E5B9)
_C2 = np.uint64(0x94D049BB133111EB)


def splitmix64(z):
    """One splitmix64 step (Steele, Lea, Flood 2014): add the golden-ratio
    increment, then the published 64-bit finalizer.  Vectorised over uint64."""
    with np.errstate(over="ignore"):
        z = np.asarray(z, dtype=np.uint64) + _PHI
        z = (z ^ (z >> np.uint64(30))) * _C1
        z = (z ^ (z >> np.uint64(27))) * _C2
        return z ^ (z >> np.uint64(31))


def noise_key(seed, request, position, vocab):
    """64-bit hash of (seed, request, position, vocab): the fields are chained
    through splitmix64, h = mix(mix(mix(mix(seed) ^ r) ^ p) ^ v)."""
    h = splitmix64(np.uint64(seed))
    h = splitmix64(h ^ np.asarray(request, dtype=np.uint64))
    h = splitmix64(h ^ np.asarray(position, dtype=np.uint64))
    return splitmix64(h ^ np.asarray(vocab, dtype=np.uint64))


def uniform_open(h):
    """Top 24 bits of the hash -> u = (k + 0.5) / 2^24, strictly inside (0, 1)."""
    k = (np.asarray(h, dtype=np.uint64) >> np.uint64(40)).astype(np.float64)
    return (k + 0.5) * (1.0 / 16777216.0)


def gumbel_noise(seed, requests, positions, vocab_size) -> np.ndarray:
    """Gumbel(0,1) noise table, g = -ln(-ln u), computed in fp64, rounded once
    to fp32.

    ``requests`` and ``positions`` are integer arrays of one shape S (position
    = absolute position of the token being sampled); the result has shape
    S + (vocab_size,).  Range: g in [-2.852, 17.329] (u is never 0 or 1).
    """
    req = np.asarray(requests, dtype=np.uint64)
    pos = np.asarray(positions, dtype=np.uint64)
    req, pos = np.broadcast_arrays(req, pos)
    shape = req.shape
    h = splitmix64(np.uint64(seed))
    h = splitmix64(h ^ req.reshape(-1))
    h = splitmix64(h ^ pos.reshape(-1))  # [rows]
    out = np.empty((h.size, vocab_size), dtype=np.float32)
    v = np.arange(vocab_size, dtype=np.uint64)[None, :]
    rows = max(1, (1 << 22) // max(1, vocab_size))  # ~4M elements per slab
    for i in range(0, h.size, rows):  # slabs keep the fp64 temporaries small
        u = uniform_open(splitmix64(h[i:i + rows, None] ^ v))
        out[i:i + rows] = (-np.log(-np.log(u))).astype(np.float32)
    return out.reshape(shape + (vocab_size,))


# ---------------------------------------------------------------------------
# Paged KV cache layout
# ---------------------------------------------------------------------------

BLOCK = 16  # tokens per KV page


@dataclass
class PagedLayout:
    """Block tables for R requests in a cache of 16-token pages.

    ``ctx`` [R] int32: L_r, verified context length (tokens already in the
    cache); the verifier's q_len rows sit at positions L_r .. L_r+q_len-1.
    ``block_table`` [R, max_blocks] int32: physical page of logical page b of
    request r, -1 where unused.  Physical pages are a seeded permutation, so
    a request's pages are not contiguous.
    """

    ctx: np.ndarray
    q_len: int
    block_table: np.ndarray
    num_blocks: int
    max_blocks: int

    def slots(self) -> np.ndarray:
        """Physical slot (page*16 + offset) of positions L_r + j, shape [R*q_len] int64."""
        R = self.ctx.shape[0]
        out = np.empty(R * self.q_len, dtype=np.int64)
        for r in range(R):
            for j in range(self.q_len):
                p = int(self.ctx[r]) + j
                out[r * self.q_len + j] = int(self.block_table[r, p // BLOCK]) * BLOCK + p % BLOCK
        return out


def paged_layout(ctx, q_len, seed, max_blocks=None, spare_blocks=0) -> PagedLayout:
    ctx = np.asarray(ctx, dtype=np.int32)
    need = [(int(c) + q_len + BLOCK - 1) // BLOCK for c in ctx]
    mb = max(need) if max_blocks is None else int(max_blocks)
    if mb < max(need):
        raise ValueError("max_blocks smaller than a request's page count")
    total = sum(need) + int(spare_blocks)
    perm = rng(seed).permutation(total).astype(np.int32)
    bt = np.full((ctx.shape[0], mb), -1, dtype=np.int32)
    o = 0
    for r, n in enumerate(need):
        bt[r, :n] = perm[o : o + n]
        o += n
    return PagedLayout(ctx=ctx, q_len=int(q_len), block_table=bt, num_blocks=total, max_blocks=mb)


# ---------------------------------------------------------------------------
# Candidates with a planted first divergence
# ---------------------------------------------------------------------------


def plant_divergence(target, d, vocab_size, seed) -> np.ndarray:
    """cand[r, j] = target[r, j] for j < d[r]; cand[r, d[r]] = some other token
    (target + 1 + U{0..V-2} mod V); positions after d[r] are random tokens.
    d[r] == K means no divergence (cand == target)."""
    target = np.asarray(target, dtype=np.int64)
    R, K = target.shape
    g = rng(seed)
    cand = g.integers(0, vocab_size, size=(R, K)).astype(np.int64)
    for r in range(R):
        dr = int(d[r])
        cand[r, :dr] = target[r, :dr]
        if dr < K:
            cand[r, dr] = (target[r, dr] + 1 + g.integers(0, vocab_size - 1)) % vocab_size
    return cand.astype(np.int32)


# ---------------------------------------------------------------------------
# Workload shapes (the configurations the method is measured on)
# ---------------------------------------------------------------------------


@dataclass(frozen=True)
class ModelShape:
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
    def qkv_out(self) -> int:
        return (self.heads + 2 * self.kv_heads) * self.head_dim


TINY = ModelShape(layers=2, hidden=256, heads=4, kv_heads=4, head_dim=64, ffn=1024, vocab=4096)
LLAMA3_8B = ModelShape(layers=32, hidden=4096, heads=32, kv_heads=8, head_dim=128, ffn=14336,
                       vocab=128256)


@dataclass
class ModelWeights:
    """Weights in the linear-layer layout [out_features, in_features]; fp32 arrays
    (tiny) or bf16 bit patterns (uint16)."""

    shape: ModelShape
    dtype: str  # "f32" or "bf16"
    embed: np.ndarray  # [V, H]
    lm_head: np.ndarray  # [V, H]
    final_norm: np.ndarray  # [H]
    layers: list = field(default_factory=list)  # dicts: attn_norm, wq, wk, wv, wo, ffn_norm, w_gate, w_up, w_down


def model_weights(shape: ModelShape, seed: int, dtype: str = "f32", layers=None, std=0.02) -> ModelWeights:
    """Random-init weights N(0, std^2); RMSNorm gains are ones."""
    H, D, F, V = shape.hidden, shape.head_dim, shape.ffn, shape.vocab
    nl = shape.layers if layers is None else layers
    mk = normal_f32 if dtype == "f32" else normal_bf16
    one = np.ones(H, dtype=np.float32)
    one = one if dtype == "f32" else bf16_bits(one)
    w = ModelWeights(shape=shape, dtype=dtype,
                     embed=mk(seed, (V, H), std, stream=(0,)),
                     lm_head=mk(seed, (V, H), std, stream=(1,)),
                     final_norm=one.copy())
    for li in range(nl):
        s = 100 + 16 * li
        w.layers.append(dict(
            attn_norm=one.copy(),
            wq=mk(seed, (shape.heads * D, H), std, stream=(s + 0,)),
            wk=mk(seed, (shape.kv_heads * D, H), std, stream=(s + 1,)),
            wv=mk(seed, (shape.kv_heads * D, H), std, stream=(s + 2,)),
            wo=mk(seed, (H, shape.heads * D), std, stream=(s + 3,)),
            ffn_norm=one.copy(),
            w_gate=mk(seed, (F, H), std, stream=(s + 4,)),
            w_up=mk(seed, (F, H), std, stream=(s + 5,)),
            w_down=mk(seed, (H, F), std, stream=(s + 6,)),
        ))
    return w


def tokens(seed, shape, vocab) -> np.ndarray:
    return rng(seed).integers(0, vocab, size=shape).astype(np.int32)


# Seeds of the page-shaped workloads (one per input, so each is reproducible alone).
SEEDS = dict(
    tiny_weights=0, tiny_prompt=1, tiny_plant=2, tiny_noise=3,
    norm_x=10, norm_gamma=11, gemm_w=12,
    attn_qkv=20, attn_len=21, attn_perm=22,
    verify_logits=30, verify_ties=31, verify_plant=32, verify_noise=33,
    pass_weights=40, pass_kv=41, pass_len=42, pass_tokens=43, pass_noise=44,
)


def context_lengths(seed, n, lo, hi) -> np.ndarray:
    """L_r ~ U{lo..hi} inclusive."""
    return rng(seed).integers(lo, hi + 1, size=n).astype(np.int32)


def fast_path_junk(shape, seed) -> np.ndarray:
    """Stand-in for fast-path KV values at the slots the verifier overwrites:
    independent values that differ from anything the verifier computes."""
    return normal_f32(seed, shape, std=3.0, stream=(7,))


def is_power_of_two(n: int) -> bool:
    return n > 0 and (n & (n - 1)) == 0


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


__all__ = [name for name in dir() if not name.startswith("_") and name not in ("annotations", "math")]


# ---------------------------------------------------------------------------
# Device-side generation for the 8B-shaped decoder (15 GB of weights, tens of
# GB of KV): seeded torch generators on the GPU, N(0, std^2) drawn in fp32 and
# rounded once to bf16.  The same tensors, copied to the host, feed the oracle.
# ---------------------------------------------------------------------------


def _torch_normal(shape, seed, stream, std, device, dtype):
    import torch

    g = torch.Generator(device=device)
    g.manual_seed((int(seed) * 1_000_003 + int(stream)) % (2 ** 63))
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


def device_model_weights(shape: ModelShape, seed: int, layers=None, device="cuda", std=0.02):
    """Random-init decoder weights on the device, bf16, in the fused layout the
    verifier uses: wqkv = [Wq; Wk; Wv] ([Hq*D + 2*Hkv*D, H]) and w_gu =
    [W_gate; W_up] ([2F, H]); RMSNorm gains are ones."""
    import torch

    nl = shape.layers if layers is None else layers
    H, D, F, V = shape.hidden, shape.head_dim, shape.ffn, shape.vocab
    bf = torch.bfloat16
    out = dict(embed=_torch_normal((V, H), seed, 0, std, device, bf),
               lm_head=_torch_normal((V, H), seed, 1, std, device, bf),
               final_norm=torch.ones(H, dtype=bf, device=device), layers=[])
    for li in range(nl):
        s = 100 + 16 * li
        out["layers"].append(dict(
            attn_norm=torch.ones(H, dtype=bf, device=device),
            wqkv=_torch_normal((shape.qkv_out, H), seed, s + 0, std, device, bf),
            wo=_torch_normal((H, shape.heads * D), seed, s + 3, std, device, bf),
            ffn_norm=torch.ones(H, dtype=bf, device=device),
            w_gu=_torch_normal((2 * F, H), seed, s + 4, std, device, bf),
            w_down=_torch_normal((H, F), seed, s + 6, std, device, bf),
        ))
    return out


def device_kv_cache(shape: ModelShape, num_blocks: int, seed: int, layers=None, device="cuda"):
    """Per-layer paged K/V caches [num_blocks, Hkv, 16, D] bf16 ~ N(0, 1): the
    context of every request (standing in for a prefill) and independent junk
    in the fast-path slots the verifier overwrites."""
    import torch

    nl = shape.layers if layers is None else layers
    caches = []
    for li in range(nl):
        k = _torch_normal((num_blocks, shape.kv_heads, BLOCK, shape.head_dim), seed, 2 * li, 1.0, device,
                          torch.bfloat16)
        v = _torch_normal((num_blocks, shape.kv_heads, BLOCK, shape.head_dim), seed, 2 * li + 1, 1.0, device,
                          torch.bfloat16)
        caches.append((k, v))
    return caches
