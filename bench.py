"""Benchmark: the batch-invariant verifier step on one MI355X.

One step = one verifier pass over W = N*K = 64*8 = 512 candidate tokens on a
Llama-3-8B-shaped decoder (32 layers, hidden 4096, 32 Q / 8 KV heads x 128,
SwiGLU FFN 14336, vocab 128256, RoPE theta 500000; bf16 random-init weights
N(0, 0.02)), contexts L_r ~ U[2048, 8192] in a paged KV cache of 16-token
pages, then Gumbel-max verification of the candidates (the KV overwrite of the
fast-path slots runs inside every layer).  Inputs are resident in HBM before
the timed region.

Prints ONE JSON line: verified tokens/s; the slowdown of the invariant pass
against the same pass with split-K GEMMs and load-adaptive attention splits
(each shape's split chosen by timing the candidates); the attention kernel's
roofline (the dominant kernel: HBM-bound, bytes = one read of each visible
K/V row, timed with HIP events on the stream it runs on); the roofline of
every kernel class of the step (each class's calls replayed as a HIP graph)
and of the whole step; and the CPU oracle timed on a bounded sample.

    python bench.py [--steps 10] [--warmup 3] [--gpus 1] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
N_REQ, K_CAND = 64, 8
CTX_LO, CTX_HI = 2048, 8192


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--layers", type=int, default=32, help=argparse.SUPPRESS)  # full model unless debugging
    p.add_argument("--micro", action="store_true",
                   help="instead of the pass: the per-kernel sweeps (RMSNorm+GEMM over M, attention over B, "
                        "Gumbel verify), one JSON line each, with rooflines, split-K/adaptive slowdowns and "
                        "oracle timings")
    p.add_argument("--iters", type=int, default=20, help="timed calls per point in --micro")
    p.add_argument("--dvr", action="store_true",
                   help="instead of the pass: decode-verify-rollback at the pass's shape (split-K fast path, K=8, "
                        "--rounds rounds) against one-token-at-a-time invariant decoding and the fast path alone")
    p.add_argument("--rounds", type=int, default=3, help="verification rounds in --dvr")
    p.add_argument("--prefill", action="store_true",
                   help="instead of the pass: causal prefill of --prompts prompts of --prompt-len tokens at the 8B "
                        "shape with the batch-invariant kernels (one forward, q_len = prompt length)")
    p.add_argument("--prompts", type=int, default=4)
    p.add_argument("--prompt-len", type=int, default=2048)
    p.add_argument("--attn-only", action="store_true",
                   help="only the pass's attention call (same contexts, pages and shapes) and a 512 MiB copy, "
                        "--iters times each: the program the HBM traffic counters are collected on")
    p.add_argument("--tree", action="store_true",
                   help="instead of the pass: tree verification by branches at the pass's shape, --branches chains "
                        "per request (each an ordinary row block; W = N*B*K rows), graph-replayed")
    p.add_argument("--branches", default="1,2,4", help="chains per request in --tree")
    p.add_argument("--gemm-only", action="store_true",
                   help="only the pass's matmuls at W = 512 rows (QKV, O + residual, gate/up + SwiGLU, down + "
                        "residual, lm_head + Gumbel epilogue), two weight copies each, --iters times each: the "
                        "program the MFMA counters are collected on")
    return p.parse_args()


TRAFFIC_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                            "attn_decode_bi_traffic.json")
ATTN_SRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "invariant_verify_verifier_amd", "csrc",
                        "attention.hip")


def _attn_source_hash():
    """SHA-256 of the attention source with comments and whitespace removed:
    it changes when the code does, not when a comment does."""
    import hashlib
    import re

    with open(ATTN_SRC) as f:
        src = f.read()
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    src = re.sub(r"\s+", " ", src).strip()
    return hashlib.sha256(src.encode()).hexdigest()


def recorded_traffic():
    """HBM bytes per attention launch from the rocprofv3 counter runs kept
    under profiles/, or None when they were taken on another version of the
    attention code."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("attention_hip_sha256") != _attn_source_hash():
        return None
    return rec.get("bytes_per_launch")


def attn_only(args):
    """The pass's attention call on its own: the 8B shapes, contexts
    U[2048, 8192] (the pass's seeds), 16-token pages, K/V ~ N(0, 1) bf16; then
    a plain 512 MiB device copy, the calibration for the byte counters."""
    import torch

    import invariant_verify_verifier_amd as biv
    import workloads as wl

    torch.cuda.set_device(0)
    sh = wl.LLAMA3_8B
    ctx = wl.context_lengths(wl.SEEDS["pass_len"], N_REQ, CTX_LO, CTX_HI)
    lay = wl.paged_layout(ctx, K_CAND, seed=wl.SEEDS["pass_len"] + 1)
    kc, vc = wl.device_kv_cache(sh, lay.num_blocks, wl.SEEDS["pass_kv"], layers=1)[0]
    q = wl._torch_normal((N_REQ * K_CAND, sh.heads * sh.head_dim), wl.SEEDS["pass_kv"], 99, 1.0, "cuda",
                         torch.bfloat16)
    out = torch.empty((N_REQ * K_CAND, sh.heads, sh.head_dim), dtype=torch.bfloat16, device="cuda")
    bt, cx = torch.from_numpy(lay.block_table).cuda(), torch.from_numpy(lay.ctx).cuda()
    ws = torch.zeros(biv.attn_workspace_bytes(N_REQ, sh.kv_heads, lay.max_blocks), dtype=torch.uint8, device="cuda")
    for _ in range(args.iters):
        biv.attn_decode_bi(q, kc, vc, bt, cx, out, K_CAND, 1.0 / math.sqrt(sh.head_dim), ws)
    src = torch.ones(512 << 20, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(args.iters):
        dst.copy_(src)
    torch.cuda.synchronize()
    algo = float(np.sum(ctx.astype(np.int64) + K_CAND)) * sh.kv_heads * sh.head_dim * 2 * 2
    print(json.dumps({"attn_only": True, "launches": args.iters, "algorithmic_bytes_per_launch": algo,
                      "copy_bytes": 512 << 20, "attention_hip_sha256": _attn_source_hash()}), flush=True)


def tree_bench(args):
    """Tree verification by branches at the pass's shape: N = 64 requests,
    K = 8, contexts U[2048, 8192], B chains per request.  Chain b of request r
    follows the target's own tokens for d[r, b] ~ U{0..K} tokens and then
    differs, so the accepted length must be max_b d[r, b] and the selected
    chain the first reaching it (checked before timing).  The step (page
    copies for every layer, the verifier step over N*B chains with the fused
    lm_head + Gumbel verification, chain selection) is captured as one HIP
    graph and replayed --steps times."""
    import torch

    from invariant_verify_verifier_amd import verifier as V
    import workloads as wl

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    Bs = [int(b) for b in args.branches.split(",")]
    extra = N_REQ * 2 * (max(Bs) - 1)
    print(f"[tree] setup: {args.layers} layers, {N_REQ} requests x K={K_CAND}, chains {Bs}", file=sys.stderr, flush=True)
    env = setup(torch, args.layers, extra_blocks=extra)
    model, caches, ctx, lay, tgt = env["model"], env["caches"], env["ctx"], env["lay"], env["tgt"]
    sh = env["sh"]
    results = {}
    for B in Bs:
        g = wl.rng(wl.SEEDS["pass_tokens"] + 10 + B)
        d = g.integers(0, K_CAND + 1, size=(N_REQ, B))
        chains = np.stack([wl.plant_divergence(tgt, d[:, b], sh.vocab, wl.SEEDS["pass_tokens"] + 20 + b)
                           for b in range(B)], axis=1)
        priv = (lay.num_blocks + np.arange(N_REQ * 2 * (B - 1))).reshape(N_REQ, B - 1, 2) if B > 1 else None
        tb = V.make_tree_batch(env["t0"], chains, ctx, lay.block_table, priv, env["noise"])
        best, acc, nxt, _ = V.verify_tree(model, tb, caches, fused_head=True)
        torch.cuda.synchronize()
        want_acc = d.max(axis=1)
        assert np.array_equal(acc.cpu().numpy(), want_acc), "accepted lengths differ from the planted ones"
        assert np.array_equal(best.cpu().numpy(), d.argmax(axis=1)), "selected chains differ"
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            V.verify_tree(model, tb, caches, fused_head=True)
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(tb.accept_len.cpu().numpy(), want_acc), "graph replay changed the decisions"
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        committed = float(np.mean(np.minimum(want_acc + 1, K_CAND)))
        results[B] = {"rows": N_REQ * B * K_CAND, "ms_per_step": round(ms, 3),
                      "verified_rows_per_s": round(N_REQ * B * K_CAND / ms * 1000, 1),
                      "mean_accepted": float(np.mean(want_acc)), "mean_committed_per_request": committed,
                      "committed_tok_per_s": round(N_REQ * committed / ms * 1000, 1)}
        print(f"[tree] B={B}: {results[B]}", file=sys.stderr, flush=True)
        del graph, tb
        torch.cuda.empty_cache()
    print(json.dumps({"tree": True, "N": N_REQ, "K": K_CAND, "layers": args.layers,
                      "workload": "Llama-3-8B-shaped verifier step over B chains per request, contexts U[2048,8192], "
                                  "chains planted with d ~ U{0..K} accepted tokens each",
                      "branches": results}), flush=True)


def gemm_only(args):
    """The pass's five matmuls at W = 512 rows with the pass's weight shapes
    (N(0, 0.02) bf16, two copies each so that consecutive calls read other
    weights, as consecutive layers do), each called --iters times in turn.
    Prints the per-call algorithmic FLOP and the mean HIP-event time of each
    matmul on the stream it runs on."""
    import torch

    import invariant_verify_verifier_amd as biv
    import workloads as wl

    torch.cuda.set_device(0)
    sh = wl.LLAMA3_8B
    W, H, F, V = N_REQ * K_CAND, sh.hidden, sh.ffn, sh.vocab
    bf = torch.bfloat16
    x = wl._torch_normal((W, H), 50, 0, 1.0, "cuda", bf)
    xf = wl._torch_normal((W, F), 50, 1, 1.0, "cuda", bf)
    res = torch.zeros((W, H), dtype=torch.float32, device="cuda")
    mk = lambda shape, s: [wl._torch_normal(shape, 51, s + c, 0.02, "cuda", bf) for c in range(2)]
    w = dict(qkv=mk((sh.qkv_out, H), 0), o=mk((H, sh.heads * sh.head_dim), 2), gu=[biv.pack_gate_up(t) for t in mk((2 * F, H), 4)],
             down=mk((H, F), 6), head=mk((V, H), 8))
    qkv = torch.empty((W, sh.qkv_out), dtype=bf, device="cuda")
    act = torch.empty((W, F), dtype=bf, device="cuda")
    noise = torch.zeros((W, V), dtype=torch.float32, device="cuda")
    cand = torch.zeros((N_REQ, K_CAND), dtype=torch.int32, device="cuda")
    tgt = torch.empty_like(cand)
    acc = torch.empty(N_REQ, dtype=torch.int32, device="cuda")
    nxt = torch.empty_like(acc)
    gws = torch.empty(biv.gumbel_workspace_bytes(W, V), dtype=torch.uint8, device="cuda")
    calls = {
        "qkv": (lambda i: biv.gemm_bi(x, w["qkv"][i % 2], qkv), 2.0 * W * H * sh.qkv_out),
        "o": (lambda i: biv.gemm_bi(x, w["o"][i % 2], res, accumulate=True), 2.0 * W * H * H),
        "gate_up_swiglu": (lambda i: biv.gemm_bi(x, w["gu"][i % 2], act, swiglu=True), 2.0 * W * H * 2 * F),
        "down": (lambda i: biv.gemm_bi(xf, w["down"][i % 2], res, accumulate=True), 2.0 * W * F * H),
        "lm_head_gumbel": (lambda i: biv.lm_head_gumbel_verify(x, w["head"][i % 2], noise, cand, tgt, acc, nxt, gws),
                           2.0 * W * H * V),
    }
    out = {}
    for name, (fn, flop) in calls.items():
        for i in range(3):
            fn(i)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(args.iters):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.iters
        out[name] = {"flop": flop, "us": round(ms * 1000, 2), "tflops": round(flop / ms / 1e9, 1),
                     "frac_of_2500": round(flop / ms / 1e9 / 2500.0, 3)}
        print(f"[gemm-only] {name}: {out[name]}", file=sys.stderr, flush=True)
    print(json.dumps({"gemm_only": True, "M": W, "calls_per_matmul": args.iters + 3, "matmuls": out}), flush=True)


MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published


class KernelCalls:
    """Records every call of the library's entry points during one eager pass,
    grouped by kernel class (installed by swapping the binding's module
    functions, which the pass looks up at call time; removed afterwards).
    ``time_classes`` then captures each class's calls, in pass order, as one
    HIP graph and times its replays with HIP events on the capturing stream:
    kernel time back to back, without the host's launch gaps that event pairs
    around short eager calls would include."""

    NAMES = ("embed_rows", "rmsnorm_bi", "gemm_bi", "rope_kv_overwrite", "attn_decode_bi",
             "lm_head_gumbel_verify")

    def __init__(self, torch):
        import invariant_verify_verifier_amd._lib as L

        self.torch, self.L = torch, L
        self.calls = {}
        self.orig = {n: getattr(L, n) for n in self.NAMES}

    @staticmethod
    def key(name, args, kw):
        if name == "gemm_bi":
            a, b = args[0], args[1]
            return ("gemm_bi", int(a.shape[0]), int(b.shape[0]), int(b.shape[1]), bool(kw.get("swiglu")),
                    bool(kw.get("accumulate")), str(args[2].dtype).replace("torch.", ""))
        return (name,)

    def __enter__(self):
        for n in self.NAMES:
            fn = self.orig[n]

            def run(*a, _n=n, _fn=fn, **k):
                self.calls.setdefault(self.key(_n, a, k), []).append((_fn, a, k))
                return _fn(*a, **k)

            setattr(self.L, n, run)
        return self

    def __exit__(self, *exc):
        for n, fn in self.orig.items():
            setattr(self.L, n, fn)

    def time_classes(self, reps=3):
        """{class: (mean ms per call, calls per pass)}."""
        n_calls = {key: len(lst) for key, lst in self.calls.items()}
        torch = self.torch
        out = {}
        for key, lst in self.calls.items():
            # a class with few calls per step is repeated so that the graph's
            # own launch cost is spread over at least 32 kernels
            lst = lst * max(1, -(-32 // len(lst)))
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for fn, a, k in lst:
                    fn(*a, **k)
            graph.replay()
            torch.cuda.synchronize()
            s = torch.cuda.Event(enable_timing=True)
            e = torch.cuda.Event(enable_timing=True)
            s.record()
            for _ in range(reps):
                graph.replay()
            e.record()
            torch.cuda.synchronize()
            out[key] = (s.elapsed_time(e) / (reps * len(lst)), n_calls[key])
            del graph
        return out


def kernel_rooflines(sh, W, ctx, timers, steps):
    """Per kernel class of the pass: algorithmic bytes and FLOPs per call, the
    bound (HBM or bf16 MFMA, whichever takes longer at the published peaks),
    the mean HIP-event time per call, and achieved / peak.  Also the whole
    step's roofline time: the sum over every call of its roofline time."""
    H, D, F, V = sh.hidden, sh.head_dim, sh.ffn, sh.vocab
    kv_tok = sh.kv_heads * D * 2  # bf16 bytes of one token's K (or V) in one layer
    out, t_roof_step = {}, 0.0
    for key, (ms, n) in sorted(timers.items(), key=lambda kv: -kv[1][0] * kv[1][1]):
        name = key[0]
        flop = 0.0
        if name == "gemm_bi":
            _, M, N, K, swiglu, acc, odt = key
            ob = 2 if odt == "bfloat16" else 4
            n_out = N // 2 if swiglu else N
            flop = 2.0 * M * N * K
            nbytes = N * K * 2 + M * K * 2 + M * n_out * ob * (2 if acc else 1)
            label = {(6144, 4096): "gemm_bi QKV", (4096, 4096): "gemm_bi O + residual",
                     (28672, 4096): "gemm_bi gate|up + SwiGLU", (4096, 14336): "gemm_bi down + residual"}.get(
                         (N, K), f"gemm_bi N={N} K={K}")
        elif name == "attn_decode_bi":
            nbytes = float(np.sum(ctx.astype(np.int64) + K_CAND)) * kv_tok * 2
            flop = 4.0 * float(np.sum(ctx.astype(np.int64) + K_CAND)) * K_CAND * sh.heads * D  # QK and PV
            label = "attn_decode_bi"
        elif name == "rmsnorm_bi":
            nbytes = W * H * (4 + 2) + H * 2
            label = "rmsnorm_bi (fp32 stream -> bf16)"
        elif name == "rope_kv_overwrite":
            nbytes = W * (sh.heads + sh.kv_heads) * D * 2 * 2 + W * sh.kv_heads * D * 2 + W * kv_tok * 2
            label = "rope_kv_overwrite"
        elif name == "embed_rows":
            nbytes = W * H * (2 + 4)
            label = "embed_rows"
        elif name == "lm_head_gumbel_verify":
            flop = 2.0 * W * H * V
            nbytes = V * H * 2 + W * V * 4 + W * H * 2
            label = "lm_head_gumbel_verify (lm_head matmul + Gumbel argmax + verify)"
        else:
            continue
        t_hbm = nbytes / (HBM_PEAK_GBS * 1e9)
        t_mfma = flop / (MFMA_BF16_PEAK_TFLOPS * 1e12)
        t_roof = max(t_hbm, t_mfma)
        per_step = n / steps
        t_roof_step += t_roof * per_step
        if t_mfma > t_hbm:
            ach, peak, unit, bound = flop / (ms / 1e3) / 1e12, MFMA_BF16_PEAK_TFLOPS, "TFLOP/s", "mfma"
        else:
            ach, peak, unit, bound = nbytes / (ms / 1e3) / 1e9, HBM_PEAK_GBS, "GB/s", "hbm"
        out[label] = {"bound": bound, "achieved": round(ach, 1), "peak": peak, "unit": unit,
                      "frac": round(ach / peak, 4), "calls_per_step": per_step, "avg_launch_ms": round(ms, 5),
                      "bytes_per_launch": nbytes, "flop_per_launch": flop,
                      "share_of_step_ms": round(ms * per_step, 4)}
    return out, t_roof_step * 1e3


class EventTimer:
    """HIP event pairs around every launch of one kernel, on its stream."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = []
        self.on = False

    def wrap(self, fn):
        def run(*a, **k):
            if not self.on:
                return fn(*a, **k)
            s = self.torch.cuda.Event(enable_timing=True)
            e = self.torch.cuda.Event(enable_timing=True)
            s.record()
            r = fn(*a, **k)
            e.record()
            self.pairs.append((s, e))
            return r

        return run

    def mean_ms(self):
        return float(np.mean([s.elapsed_time(e) for s, e in self.pairs])) if self.pairs else float("nan")


def setup(torch, n_layers, extra_blocks=0):
    import workloads as wl
    from invariant_verify_verifier_amd import verifier as V

    sh = wl.LLAMA3_8B
    ctx = wl.context_lengths(wl.SEEDS["pass_len"], N_REQ, CTX_LO, CTX_HI)
    lay = wl.paged_layout(ctx, K_CAND, seed=wl.SEEDS["pass_len"] + 1)
    dw = wl.device_model_weights(sh, wl.SEEDS["pass_weights"], layers=n_layers)
    caches = wl.device_kv_cache(sh, lay.num_blocks + extra_blocks, wl.SEEDS["pass_kv"], layers=n_layers)
    shape = V.Shape(n_layers, sh.hidden, sh.heads, sh.kv_heads, sh.head_dim, sh.ffn, sh.vocab, sh.eps,
                    sh.rope_theta)
    model = V.VerifierModel(shape, torch.bfloat16, dw["layers"], dw["embed"], dw["lm_head"], dw["final_norm"],
                            max_pos=16384)
    t0 = wl.tokens(wl.SEEDS["pass_tokens"], (N_REQ,), sh.vocab)
    cand0 = wl.tokens(wl.SEEDS["pass_tokens"] + 1, (N_REQ, K_CAND), sh.vocab)
    pos = ctx[:, None] + np.arange(K_CAND)[None, :] + 1
    noise = wl.gumbel_noise(wl.SEEDS["pass_noise"], np.repeat(np.arange(N_REQ), K_CAND).reshape(N_REQ, K_CAND),
                            pos, sh.vocab)
    # candidates: the target's own tokens up to a planted first divergence
    # d ~ U{0..K}
    tgt = V.self_consistent_candidates(model, t0, ctx, lay.block_table, noise, caches, K_CAND, first=cand0)
    d = wl.rng(wl.SEEDS["pass_tokens"] + 2).integers(0, K_CAND + 1, size=N_REQ)
    cand = wl.plant_divergence(tgt, d, sh.vocab, wl.SEEDS["pass_tokens"] + 2)
    batch = V.make_batch(t0, cand, ctx, lay.block_table, noise)
    return dict(sh=sh, ctx=ctx, lay=lay, dw=dw, caches=caches, model=model, batch=batch, d=d, t0=t0, cand=cand,
                noise=noise, tgt=tgt)


def time_graph(torch, model, batch, caches, steps, warmup, **kw):
    """The pass captured as one HIP graph: warm-up replays, then `steps`
    replays between two events; ms per replay."""
    graph = model.capture(batch, caches, **kw)
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        graph.replay()
    end.record()
    torch.cuda.synchronize()
    del graph
    return start.elapsed_time(end) / steps


def gpu_state_under_load(torch, replay, limit_s=20):
    """rocm-smi's clocks, socket power and performance level, read while the
    pass replays (untimed, after the timed region); None where the tool is
    missing or fails."""
    import shutil
    import subprocess
    import threading

    tool = shutil.which("rocm-smi")
    if tool is None:
        return None
    out = {}

    def sample():
        try:
            p = subprocess.run([tool, "--showclocks", "--showpower", "--showperflevel", "--json"],
                               capture_output=True, text=True, timeout=limit_s)
            out["text"] = p.stdout
        except (OSError, subprocess.SubprocessError) as e:
            out["error"] = repr(e)

    th = threading.Thread(target=sample)
    th.start()
    while th.is_alive():  # the tool's own time limit ends this loop
        replay()
        torch.cuda.synchronize()
    th.join()
    try:
        cards = json.loads(out.get("text", ""))
    except ValueError:
        return {"error": out.get("error", "unparsed rocm-smi output")}
    keep = {}
    for card, fields in cards.items():
        if isinstance(fields, dict):
            keep[card] = {k.strip(" :"): v for k, v in fields.items()
                          if any(w in k.lower() for w in ("clk", "power", "performance"))}
    return {"tool": "rocm-smi --showclocks --showpower --showperflevel", "sampled": "during untimed graph replays",
            "cards": keep}


def _dvr_event_ms(fn, iters=5, warmup=2):
    from invariant_verify_verifier_amd.dvr import _event_ms

    return _event_ms(fn, iters=iters, warmup=warmup)


def time_passes(torch, model, batch, caches, steps, **kw):
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        model.verify(batch, caches, **kw)
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def _host_cpu():
    """The host's CPU model (lscpu's "Model name", else /proc/cpuinfo), the
    cores this process may run on, and the logical CPUs the host reports."""
    import platform
    import subprocess

    model = None
    try:
        p = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10)
        for ln in p.stdout.splitlines():
            if ln.strip().lower().startswith("model name"):
                model = ln.split(":", 1)[1].strip()
                break
    except (OSError, subprocess.SubprocessError):
        pass
    if model is None:
        try:
            with open("/proc/cpuinfo") as f:
                for ln in f:
                    if ln.lower().startswith("model name"):
                        model = ln.split(":", 1)[1].strip()
                        break
        except OSError:
            model = platform.processor() or None
    return {"model": model, "affinity_cores": len(os.sched_getaffinity(0)), "nproc": os.cpu_count()}


def cpu_baseline(torch, env, n_layers, sample_layers=3):
    """The oracle, untouched, on a bounded sample of the same workload: the
    first `sample_layers` decoder layers over all 512 rows, then the final
    norm, lm_head and verify; extrapolated to the full depth as
    n_layers * mean(t_layer) + t_head per pass.  Run with NumPy's BLAS on
    every core this process may use, then once more on one thread for one
    layer of the sample (the rate per row is the same work per row)."""
    import oracle
    import workloads as wl
    from threadpoolctl import threadpool_info, threadpool_limits

    sh, dw, lay, ctx = env["sh"], env["dw"], env["lay"], env["ctx"]
    n = N_REQ
    H, D, F = sh.hidden, sh.head_dim, sh.ffn
    q, kv = sh.heads * D, sh.kv_heads * D

    def f64(t):
        b = t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)

    host = _host_cpu()
    cores = host["affinity_cores"]
    limiter = threadpool_limits(limits=cores)
    blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    used = sorted({int(b) for b in lay.block_table[:n].ravel() if b >= 0})
    remap = {b: i for i, b in enumerate(used)}
    bt = np.vectorize(lambda b: remap.get(int(b), -1))(lay.block_table[:n]).astype(np.int32)
    toks = np.concatenate([env["t0"][:n, None], env["cand"][:n, :K_CAND - 1]], axis=1)
    lm = f64(dw["lm_head"])
    t_layers = []
    one_thread = None
    for li in range(min(sample_layers, n_layers)):
        Ld = dw["layers"][li]
        wqkv, wgu = f64(Ld["wqkv"]), f64(Ld["w_gu"])
        layer = dict(attn_norm=f64(Ld["attn_norm"]), wq=wqkv[:q], wk=wqkv[q:q + kv], wv=wqkv[q + kv:],
                     wo=f64(Ld["wo"]), ffn_norm=f64(Ld["ffn_norm"]), w_gate=wgu[:F], w_up=wgu[F:],
                     w_down=f64(Ld["w_down"]))
        ow = dict(shape=wl.ModelShape(1, H, sh.heads, sh.kv_heads, D, F, sh.vocab, sh.eps, sh.rope_theta),
                  embed=f64(dw["embed"]), lm_head=lm[:1], final_norm=f64(dw["final_norm"]), layers=[layer])
        kc = f64(env["caches"][li][0][used])
        vc = f64(env["caches"][li][1][used])
        # one layer: the oracle's decoder forward with a 1-layer model and a
        # throwaway one-row head, timed apart from the real head
        t = time.perf_counter()
        oracle.decoder_forward(ow, toks, ctx[:n], [kc], [vc], bt)
        t_layers.append(time.perf_counter() - t)
        if li == 0:
            # the same layer on one thread, over the first 8 requests (64 rows)
            n1 = 8
            used1 = sorted({int(b) for b in lay.block_table[:n1].ravel() if b >= 0})
            kc1 = f64(env["caches"][li][0][used1])
            vc1 = f64(env["caches"][li][1][used1])
            remap1 = {b: i for i, b in enumerate(used1)}
            bt1 = np.vectorize(lambda b: remap1.get(int(b), -1))(lay.block_table[:n1]).astype(np.int32)
            with threadpool_limits(limits=1):
                t = time.perf_counter()
                oracle.decoder_forward(ow, toks[:n1], ctx[:n1], [kc1], [vc1], bt1)
                t1 = time.perf_counter() - t
            one_thread = {"rows": n1 * K_CAND, "t_layer_s": round(t1, 3),
                          "rows_per_s_per_layer": round(n1 * K_CAND / t1, 3)}
            del kc1, vc1
        del kc, vc, wqkv, wgu, layer
    x = wl.normal_f32(1, (n * K_CAND, H)).astype(np.float64)
    t = time.perf_counter()
    logits = oracle.linear(oracle.rmsnorm(x, f64(dw["final_norm"]), sh.eps), lm)
    oracle.gumbel_verify(logits.astype(np.float32).reshape(n, K_CAND, -1), env["noise"][:n], env["cand"][:n])
    t_head = time.perf_counter() - t
    t_layer = float(np.mean(t_layers))
    t_pass = n_layers * t_layer + t_head
    limiter.restore_original_limits()
    out = {"value": round(n * K_CAND / t_pass, 3), "unit": "verified tok/s", "cores": int(cores),
           "kind": "oracle",
           "sample": f"{len(t_layers)} of {n_layers} layers + lm_head/verify over all {n * K_CAND} rows, fp64; "
                     f"t_layer={t_layer:.2f}s (mean) t_head={t_head:.2f}s; pass = {n_layers}*t_layer + t_head "
                     f"(extrapolated); matmuls on NumPy's BLAS with {blas_threads} threads, the attention's "
                     f"per-row loop in one Python thread",
           "host_cpu": host, "blas_threads": int(blas_threads)}
    if one_thread is not None:
        one_thread["pass_extrapolated_tok_s"] = round(
            one_thread["rows_per_s_per_layer"] / n_layers, 4)
        one_thread["note"] = ("layer 0 over the first 8 requests on one thread; pass = rows / (32 * t_layer), "
                              "head not included")
        out["single_thread"] = one_thread
    return out


# ---------------------------------------------------------------------------
# --micro: the kernel-level workloads (RMSNorm+GEMM microbench, attention at
# batch 1..256 with contexts U[512, 32768], Gumbel verify at [64, 8, 128256])
# ---------------------------------------------------------------------------

MFMA_PEAK_TFLOPS = 2500.0


def _event_times(torch, fn, iters, warmup=5, pre=None):
    """Median and p90 (ms) of per-call HIP event pairs on the current stream;
    `pre` runs before each call, outside the pair."""
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    pairs = []
    for i in range(iters):
        if pre is not None:
            pre()
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        fn(i)
        e.record()
        pairs.append((s, e))
    torch.cuda.synchronize()
    t = np.sort([s.elapsed_time(e) for s, e in pairs])
    return float(np.median(t)), float(t[min(len(t) - 1, int(math.ceil(0.9 * len(t))) - 1)])


def _f64_bf16(torch, t):
    b = t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def micro_norm_gemm(torch, biv, iters):
    """RMSNorm over 4096 (bf16 gamma ~ N(1, 0.1)) feeding a GEMM with a bf16
    weight [14336, 4096] ~ N(0, 0.02); M in 1..512; four weight copies rotate
    so that the weight is read from HBM each call."""
    import oracle
    import workloads as wl

    H, N, eps = 4096, 14336, 1e-6
    x_all = torch.from_numpy(wl.normal_bf16(wl.SEEDS["norm_x"], (512, H)).view(np.int16)).cuda().view(torch.bfloat16)
    gamma = torch.from_numpy(wl.normal_bf16(wl.SEEDS["norm_gamma"], (H,), std=0.1, mean=1.0).view(np.int16)).cuda()
    gamma = gamma.view(torch.bfloat16)
    ws = [wl._torch_normal((N, H), wl.SEEDS["gemm_w"], i, 0.02, "cuda", torch.bfloat16) for i in range(4)]
    points = []
    for M in [1 << i for i in range(10)]:
        x = x_all[:M]
        h = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
        out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

        def run_bi(i):
            biv.rmsnorm_bi(x, gamma, h, eps)
            biv.gemm_bi(h, ws[i % 4], out)

        def run_sk(sp, wsk):
            def run(i):
                biv.rmsnorm_bi(x, gamma, h, eps)
                biv.gemm_splitk(h, ws[i % 4], out, sp, wsk)
            return run

        t_bi, p90 = _event_times(torch, run_bi, iters)
        # the comparison: split-K timed at 1, 2, 4 and 8 splits of K, the fastest kept (1 split is gemm_bi)
        t_by = {}
        for sp in (1, 2, 4, 8):
            wsk = torch.empty(max(biv.splitk_workspace_bytes(M, N, sp), 16), dtype=torch.uint8, device="cuda")
            t_by[sp] = _event_times(torch, run_sk(sp, wsk), iters)[0]
            del wsk
        sp = min(t_by, key=t_by.get)
        t_sk = t_by[sp]
        byts = N * H * 2 + M * H * 2 * 2 + M * N * 2
        flops = 2.0 * M * N * H
        t_roof = max(byts / (HBM_PEAK_GBS * 1e9), flops / (MFMA_PEAK_TFLOPS * 1e12)) * 1e3
        points.append({"M": M, "ms": round(t_bi, 5), "ms_p90": round(p90, 5),
                       "bound": "hbm" if byts / (HBM_PEAK_GBS * 1e9) >= flops / (MFMA_PEAK_TFLOPS * 1e12) else "mfma",
                       "roofline_ms": round(t_roof, 5), "frac": round(t_roof / t_bi, 4),
                       "splitk_splits": sp, "splitk_ms": round(t_sk, 5), "slowdown_vs_splitk": round(t_bi / t_sk, 4),
                       "splitk_ms_by_splits": {str(k): round(v, 5) for k, v in t_by.items()},
                       "splitk_auto_splits": biv.splitk_auto_splits(M, N, H)})
        print(f"[micro] rmsnorm+gemm M={M}: {t_bi * 1e3:.1f} us (roof {t_roof * 1e3:.1f}), split-K best x{sp} "
              f"{t_sk * 1e3:.1f} us", file=sys.stderr, flush=True)
    # oracle: the same two steps in fp64 on the host
    w64 = _f64_bf16(torch, ws[0])
    g64 = _f64_bf16(torch, gamma)
    x64 = _f64_bf16(torch, x_all)
    cpu = []
    for M in (1, 64, 512):
        t = time.perf_counter()
        oracle.linear(oracle.rmsnorm(x64[:M], g64, eps), w64)
        cpu.append({"M": M, "s": round(time.perf_counter() - t, 4)})
    return {"workload": "rmsnorm_bi + gemm_bi: x [M,4096] bf16 ~N(0,1), gamma ~N(1,0.1), W [14336,4096] bf16 "
                        "~N(0,0.02), bf16 out; 4 rotating weight copies",
            "points": points, "cpu_oracle": {"kind": "oracle", "fp64": True, "threads": _threads(), "runs": cpu}}


def micro_attention(torch, biv, iters):
    """Decode attention, 32 Q / 8 KV heads x 128, 16-token pages placed by a
    seeded permutation, contexts U[512, 32768]; batch B takes the first B
    requests; q_len 1 (decode) and 8 (verify-shaped).  A 512 MiB write before
    every timed call evicts the 256 MB last-level cache."""
    import oracle
    import workloads as wl

    Rmax, Hq, Hkv, D = 256, 32, 8, 128
    ctx_all = wl.context_lengths(wl.SEEDS["attn_len"], Rmax, 512, 32768)
    lay = wl.paged_layout(ctx_all, 8, seed=wl.SEEDS["attn_perm"])
    kc = wl._torch_normal((lay.num_blocks, Hkv, 16, D), wl.SEEDS["attn_qkv"], 1, 1.0, "cuda", torch.bfloat16)
    vc = wl._torch_normal((lay.num_blocks, Hkv, 16, D), wl.SEEDS["attn_qkv"], 2, 1.0, "cuda", torch.bfloat16)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    bt_all = torch.from_numpy(lay.block_table).cuda()
    cx_all = torch.from_numpy(lay.ctx).cuda()
    scale = 1.0 / math.sqrt(D)
    out = {}
    for q_len in (1, 8):
        q_all = wl._torch_normal((Rmax * q_len, Hq * D), wl.SEEDS["attn_qkv"], 10 + q_len, 1.0, "cuda",
                                 torch.bfloat16)
        o = torch.empty((Rmax * q_len, Hq, D), dtype=torch.bfloat16, device="cuda")
        points = []
        for B in [1 << i for i in range(9)]:
            bt, cx, q = bt_all[:B].contiguous(), cx_all[:B].contiguous(), q_all[:B * q_len]
            ob = o[:B * q_len]
            wsb = torch.empty(biv.attn_workspace_bytes(B, Hkv, lay.max_blocks), dtype=torch.uint8, device="cuda")
            run_bi = lambda i: biv.attn_decode_bi(q, kc, vc, bt, cx, ob, q_len, scale, wsb)
            t_bi, p90 = _event_times(torch, run_bi, iters, pre=flush.zero_)
            # the comparison: the load-adaptive split, half of it and twice it (multiples of 256 tokens
            # within the block table's capacity), each timed, the fastest kept
            auto = biv.attn_adaptive_split(B, Hkv, lay.max_blocks)
            cap = -(-lay.max_blocks * 16 // 256) * 256
            t_by = {}
            for sp_tok in sorted({max(256, auto // 2 // 256 * 256), auto, min(cap, auto * 2)}):
                wsa = torch.empty(max(biv.attn_workspace_bytes(B, Hkv, lay.max_blocks, sp_tok), 16),
                                  dtype=torch.uint8, device="cuda")
                run_ad = lambda i: biv.attn_decode_adaptive(q, kc, vc, bt, cx, ob, q_len, scale, wsa,
                                                            split_tokens=sp_tok)
                t_by[sp_tok] = _event_times(torch, run_ad, iters, pre=flush.zero_)[0]
                del wsa
            split = min(t_by, key=t_by.get)
            t_ad = t_by[split]
            byts = float((ctx_all[:B].astype(np.int64) + q_len).sum()) * Hkv * D * 2 * 2
            t_roof = byts / (HBM_PEAK_GBS * 1e9) * 1e3
            points.append({"B": B, "ms": round(t_bi, 5), "ms_p90": round(p90, 5), "bytes": byts,
                           "GBps": round(byts / (t_bi * 1e-3) / 1e9, 1), "roofline_ms": round(t_roof, 5),
                           "frac": round(t_roof / t_bi, 4), "adaptive_split": split, "adaptive_ms": round(t_ad, 5),
                           "slowdown_vs_adaptive": round(t_bi / t_ad, 4), "adaptive_auto_split": auto,
                           "adaptive_ms_by_split": {str(k): round(v, 5) for k, v in t_by.items()}})
            print(f"[micro] attention q_len={q_len} B={B}: {t_bi * 1e3:.1f} us ({t_roof / t_bi:.2f} of HBM), "
                  f"adaptive best split {split}: {t_ad * 1e3:.1f} us", file=sys.stderr, flush=True)
        out[f"q_len={q_len}"] = points
    # oracle: decode (q_len 1) at B = 1 and 16, on host copies of the pages used
    cpu = []
    q1 = _f64_bf16(torch, wl._torch_normal((16, Hq * D), wl.SEEDS["attn_qkv"], 11, 1.0, "cuda", torch.bfloat16))
    for B in (1, 16):
        used = sorted({int(b) for b in lay.block_table[:B].ravel() if b >= 0})
        remap = {b: i for i, b in enumerate(used)}
        idx = torch.tensor(used, device="cuda")
        k64, v64 = _f64_bf16(torch, kc[idx]), _f64_bf16(torch, vc[idx])
        bt64 = np.vectorize(lambda b: remap.get(int(b), -1))(lay.block_table[:B]).astype(np.int32)
        t = time.perf_counter()
        oracle.attention(q1[:B].reshape(B, Hq, D), k64, v64, bt64, ctx_all[:B], 1, scale)
        cpu.append({"B": B, "q_len": 1, "s": round(time.perf_counter() - t, 4)})
        del k64, v64
    return {"workload": "attn_decode_bi: Q 32 heads, K/V 8 heads x 128 bf16 ~N(0,1), 16-token pages (seeded "
                        "permutation), contexts U[512,32768], batch = first B of 256 requests; cache flushed "
                        "before each call",
            "points": out, "cpu_oracle": {"kind": "oracle", "fp64": True, "threads": _threads(), "runs": cpu}}


def micro_verify(torch, biv, iters):
    """Gumbel verify on logits [64, 8, 128256] ~ N(0, 9) fp32 with planted
    near-ties, noise from the seeded hash, candidates with a first divergence
    d ~ U{0..8}."""
    import oracle
    import workloads as wl

    R, K, V = 64, 8, 128256
    logits = wl.normal_f32(wl.SEEDS["verify_logits"], (R, K, V), std=3.0)
    pos = np.arange(K)[None, :] + 1 + wl.context_lengths(wl.SEEDS["verify_plant"], R, 2048, 8192)[:, None]
    noise = wl.gumbel_noise(wl.SEEDS["verify_noise"], np.repeat(np.arange(R), K).reshape(R, K), pos, V)
    tgt, _, _ = oracle.gumbel_verify(logits, noise, np.zeros((R, K), np.int32))
    d = wl.rng(wl.SEEDS["verify_plant"]).integers(0, K + 1, size=R)
    cand = wl.plant_divergence(tgt, d, V, wl.SEEDS["verify_plant"])
    t = time.perf_counter()
    o_tgt, o_acc, o_next = oracle.gumbel_verify(logits, noise, cand)
    t_cpu = time.perf_counter() - t
    lg = torch.from_numpy(logits.reshape(R * K, V)).cuda()
    nz = torch.from_numpy(noise.reshape(R * K, V)).cuda()
    cd = torch.from_numpy(cand).cuda()
    tg = torch.empty((R, K), dtype=torch.int32, device="cuda")
    ac = torch.empty(R, dtype=torch.int32, device="cuda")
    nx = torch.empty(R, dtype=torch.int32, device="cuda")
    run = lambda i: biv.gumbel_verify(lg, nz, cd, tg, ac, nx)
    t_gpu, p90 = _event_times(torch, run, iters)
    exact = bool(np.array_equal(tg.cpu().numpy(), o_tgt) and np.array_equal(ac.cpu().numpy(), o_acc)
                 and np.array_equal(nx.cpu().numpy(), o_next))
    byts = 2.0 * R * K * V * 4
    t_roof = byts / (HBM_PEAK_GBS * 1e9) * 1e3
    print(f"[micro] gumbel_verify: {t_gpu * 1e3:.1f} us (roof {t_roof * 1e3:.1f}), oracle {t_cpu:.2f} s",
          file=sys.stderr, flush=True)
    # Gumbel top-8 of the same rows (k draws without replacement per row)
    KT = 8
    t = time.perf_counter()
    o_idx, o_sc = oracle.gumbel_topk(logits.reshape(R * K, V), noise.reshape(R * K, V), KT)
    t_cpu_k = time.perf_counter() - t
    ix = torch.empty((R * K, KT), dtype=torch.int32, device="cuda")
    sc = torch.empty((R * K, KT), dtype=torch.float32, device="cuda")
    t_gpu_k, p90_k = _event_times(torch, lambda i: biv.gumbel_topk(lg, nz, ix, sc), iters)
    exact_k = bool(np.array_equal(ix.cpu().numpy(), o_idx) and
                   np.array_equal(sc.cpu().numpy().view(np.uint32), o_sc.astype(np.float32).view(np.uint32)))
    print(f"[micro] gumbel_topk k={KT}: {t_gpu_k * 1e3:.1f} us, oracle {t_cpu_k:.2f} s", file=sys.stderr, flush=True)
    return {"workload": "gumbel_verify: logits [64,8,128256] fp32 ~N(0,9), seeded Gumbel noise table, planted "
                        "first divergence d ~ U{0..8}",
            "ms": round(t_gpu, 5), "ms_p90": round(p90, 5), "roofline_ms": round(t_roof, 5),
            "frac": round(t_roof / t_gpu, 4), "rows_per_s": round(R * K / (t_gpu * 1e-3), 1),
            "bitwise_equal_to_oracle": exact,
            "cpu_oracle": {"kind": "oracle", "threads": _threads(), "s": round(t_cpu, 4),
                           "rows_per_s": round(R * K / t_cpu, 1)},
            "topk": {"k": KT, "ms": round(t_gpu_k, 5), "ms_p90": round(p90_k, 5), "roofline_ms": round(t_roof, 5),
                     "frac": round(t_roof / t_gpu_k, 4), "bitwise_equal_to_oracle": exact_k,
                     "cpu_oracle": {"kind": "oracle", "threads": _threads(), "s": round(t_cpu_k, 4)}}}


def _threads():
    from threadpoolctl import threadpool_info

    return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])


def micro(args):
    import torch

    import invariant_verify_verifier_amd as biv

    assert torch.cuda.is_available(), "bench.py --micro needs a GPU"
    torch.cuda.set_device(0)
    for name, fn in (("rmsnorm+gemm", micro_norm_gemm), ("attention", micro_attention),
                     ("gumbel_verify", micro_verify)):
        print(f"[micro] {name}", file=sys.stderr, flush=True)
        res = fn(torch, biv, args.iters)
        print(json.dumps({"micro": name, **res}), flush=True)
        torch.cuda.empty_cache()


def prefill_bench(args):
    """Causal prefill with the batch-invariant kernels at the 8B shape: R
    prompts of P tokens from context 0 in one forward (q_len = P; attention
    in 32-row blocks, each with the keys up to its own last row), writing the
    prompts' K/V.  Its rows are bit for bit those of decoding the prompt one
    token at a time (tested on the 2-layer slice)."""
    import torch

    import workloads as wl
    from invariant_verify_verifier_amd import verifier as V

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    sh, R, P = wl.LLAMA3_8B, args.prompts, args.prompt_len
    print(f"[bench] prefill setup: {args.layers} layers, {R} prompts x {P} tokens", file=sys.stderr, flush=True)
    dw = wl.device_model_weights(sh, wl.SEEDS["pass_weights"], layers=args.layers)
    shape = V.Shape(args.layers, sh.hidden, sh.heads, sh.kv_heads, sh.head_dim, sh.ffn, sh.vocab, sh.eps,
                    sh.rope_theta)
    model = V.VerifierModel(shape, torch.bfloat16, dw["layers"], dw["embed"], dw["lm_head"], dw["final_norm"],
                            max_pos=max(16384, P + 16))
    ctx = np.zeros(R, np.int32)
    lay = wl.paged_layout(ctx, P, seed=wl.SEEDS["pass_len"] + 3)
    caches = model.alloc_kv(lay.num_blocks)
    pos = np.tile(np.arange(P, dtype=np.int32), R)
    rows = np.repeat(np.arange(R), P)
    slots = lay.block_table[rows, pos // 16].astype(np.int64) * 16 + pos % 16
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    toks, pos_d, ctx_d, bt, sl = (dev(wl.tokens(wl.SEEDS["pass_tokens"] + 5, (R * P,), sh.vocab)), dev(pos),
                                  dev(ctx), dev(lay.block_table), dev(slots))
    run = lambda: model.forward(toks, pos_d, ctx_d, P, bt, sl, caches)
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        run()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    # the lm_head over every prompt row is part of this forward (logits of all rows)
    flops = 2.0 * R * P * (args.layers * (sh.hidden * (sh.heads + 2 * sh.kv_heads) * sh.head_dim
                                          + sh.heads * sh.head_dim * sh.hidden + 3 * sh.hidden * sh.ffn)
                           + sh.hidden * sh.vocab)
    attn_flops = 4.0 * args.layers * R * sh.heads * sh.head_dim * (P * (P + 1) / 2)
    line = {"metric": "prefill tokens/s (1 GPU)", "value": round(R * P / (ms / 1e3), 1), "unit": "prompt tok/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 3),
            "higher_is_better": True, "dtype": "bf16",
            "data": "synthetic (seeded random-init weights, random prompt tokens)",
            "config": {"workload": f"Llama-3-8B-shaped causal prefill ({args.layers} layers), {R} prompts x {P} tokens "
                                   "from context 0, batch-invariant kernels, logits of every row",
                       "prompts": R, "prompt_len": P},
            "mfma_tflops": round((flops + attn_flops) / (ms / 1e3) / 1e12, 1)}
    print(json.dumps(line), flush=True)


def dvr_bench(args):
    """Decode-verify-rollback (LLM-42 post, paragraphs 3-4) at the pass's
    shape: N = 64 requests, K = 8, contexts U[2048, 8192].  Three ways to
    produce the same number of tokens per request, timed with HIP events:
    the fast path alone (split-K GEMMs + adaptive attention splits, one token
    per forward, not batch invariant), decode-verify-rollback (K fast-path
    tokens, then one invariant verifier pass over all N*K), and
    one-token-at-a-time decoding with the invariant kernels.  The committed
    streams of the last two must be equal.  Gumbel noise for every (request,
    position) the run can reach is made before the timed region."""
    import torch

    import workloads as wl
    from invariant_verify_verifier_amd import dvr as D
    from invariant_verify_verifier_amd import verifier as V

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    sh, K, R = wl.LLAMA3_8B, K_CAND, N_REQ
    n_tok = args.rounds * K
    # every sampled position lies in ctx+1 .. ctx+n_tok: a round starts after
    # at most (rounds-1)*K committed tokens and samples K more
    span = n_tok
    ctx = wl.context_lengths(wl.SEEDS["pass_len"], R, CTX_LO, CTX_HI)
    lay = wl.paged_layout(ctx, n_tok + K, seed=wl.SEEDS["pass_len"] + 1)
    print(f"[bench] dvr setup: {args.layers} layers, {R} requests, K={K}, {args.rounds} rounds", file=sys.stderr,
          flush=True)
    dw = wl.device_model_weights(sh, wl.SEEDS["pass_weights"], layers=args.layers)
    caches = wl.device_kv_cache(sh, lay.num_blocks, wl.SEEDS["pass_kv"], layers=args.layers)
    shape = V.Shape(args.layers, sh.hidden, sh.heads, sh.kv_heads, sh.head_dim, sh.ffn, sh.vocab, sh.eps,
                    sh.rope_theta)
    model = V.VerifierModel(shape, torch.bfloat16, dw["layers"], dw["embed"], dw["lm_head"], dw["final_norm"],
                            max_pos=16384)
    t0 = wl.tokens(wl.SEEDS["pass_tokens"], (R,), sh.vocab)
    table = torch.empty((R, span, sh.vocab), dtype=torch.float32, device="cuda")
    for i in range(span):
        table[:, i] = torch.from_numpy(wl.gumbel_noise(wl.SEEDS["pass_noise"], np.arange(R), ctx + 1 + i, sh.vocab))
    print("[bench] dvr noise ready", file=sys.stderr, flush=True)
    ctx_of = np.asarray(ctx, np.int64)

    def noise_fn(req, pos):
        req = np.asarray(req, np.int64)
        off = np.asarray(pos, np.int64) - ctx_of[req] - 1
        return table[torch.from_numpy(req).cuda(), torch.from_numpy(off).cuda()]

    dvr = D.DecodeVerifyRollback(model, caches, lay.block_table, K, noise_fn, fast="split")

    def timed(fn):
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        out = fn()
        end.record()
        torch.cuda.synchronize()
        return out, start.elapsed_time(end) / 1e3

    # warm-up: workspaces and buffers for both row counts
    dvr.sequential(t0, ctx, 1)
    dvr.sequential(t0, ctx, 1, **dvr.fast_kw)
    dvr.verify(t0, np.zeros((R, K), np.int32), ctx)
    print("[bench] dvr warm-up done", file=sys.stderr, flush=True)
    inv_seq, t_inv = timed(lambda: dvr.sequential(t0, ctx, n_tok))
    print(f"[bench] invariant decode: {t_inv:.3f} s", file=sys.stderr, flush=True)
    fast_seq, t_fast = timed(lambda: dvr.sequential(t0, ctx, n_tok, **dvr.fast_kw))
    print(f"[bench] fast-path decode: {t_fast:.3f} s", file=sys.stderr, flush=True)
    dvr.stats = D.RoundStats()

    hist, t_dvr = timed(lambda: dvr.run(t0, ctx, args.rounds))
    print(f"[bench] decode-verify-rollback: {t_dvr:.3f} s", file=sys.stderr, flush=True)
    n_dvr = sum(len(h) for h in hist)
    equal = all(np.array_equal(np.asarray(h[:n_tok], np.int32), inv_seq[r, :len(h[:n_tok])])
                for r, h in enumerate(hist))
    v_dvr, v_inv, v_fast = n_dvr / t_dvr, R * n_tok / t_inv, R * n_tok / t_fast
    line = {
        "metric": "decode-verify-rollback committed tokens/s (1 GPU)",
        "value": round(v_dvr, 2),
        "unit": "committed tok/s",
        "n_gpus": 1,
        "steps": args.rounds,
        "higher_is_better": True,
        "dtype": "bf16",
        "data": "synthetic (seeded random-init weights and KV of the stated shapes)",
        "config": {"workload": f"Llama-3-8B-shaped decoder ({args.layers} layers), N = {R} requests, K = {K}, "
                               "contexts U[2048,8192], fast path split-K + adaptive attention splits",
                   "rounds": args.rounds, "tokens_per_request_baselines": n_tok},
        "acceptance": round(dvr.stats.acceptance(K), 4),
        "tokens_per_round": round(dvr.stats.tokens_per_round(), 3),
        "committed_tokens": n_dvr,
        "streams_equal_invariant_decode": bool(equal),
        "all_invariant_decode_tok_s": round(v_inv, 2),
        "fast_path_decode_tok_s": round(v_fast, 2),
        "fast_path_streams_equal_invariant": int(sum(np.array_equal(fast_seq[r], inv_seq[r]) for r in range(R))),
        "dvr_vs_all_invariant": round(v_dvr / v_inv, 4),
    }
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.micro and args.gpus == 1:
        micro(args)
        return
    if args.prefill and args.gpus == 1:
        prefill_bench(args)
        return
    if args.dvr and args.gpus == 1:
        dvr_bench(args)
        return
    if args.attn_only and args.gpus == 1:
        attn_only(args)
        return
    if args.gemm_only and args.gpus == 1:
        gemm_only(args)
        return
    if args.tree and args.gpus == 1:
        tree_bench(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the verifier step would shard by request, with no traffic between GPUs)",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import invariant_verify_verifier_amd as biv

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    print(f"[bench] setup: {args.layers} layers, {N_REQ}x{K_CAND} rows", file=sys.stderr, flush=True)
    env = setup(torch, args.layers)
    model, batch, caches, ctx = env["model"], env["batch"], env["caches"], env["ctx"]
    timer = EventTimer(torch)
    attn = timer.wrap(biv.attn_decode_bi)
    for i in range(args.warmup):
        model.verify(batch, caches, attn_fn=attn)
    torch.cuda.synchronize()
    acc = batch.accept_len.cpu().numpy()
    assert np.array_equal(acc, env["d"]), f"planted divergence not recovered: {acc} vs {env['d']}"
    tgt_bi = batch.target.cpu().numpy().copy()
    acc_bi = batch.accept_len.cpu().numpy().copy()
    nxt_bi = batch.next_token.cpu().numpy().copy()
    # the step as timed: lm_head and Gumbel verification fused (no logits in
    # HBM); its decisions must be those of the unfused step, bit for bit
    model.verify(batch, caches, fused_head=True)
    torch.cuda.synchronize()
    for got, ref, what in ((batch.target, tgt_bi, "targets"), (batch.accept_len, acc_bi, "accept_len"),
                           (batch.next_token, nxt_bi, "next_token")):
        assert np.array_equal(got.cpu().numpy(), ref), f"fused head changed {what}"
    # eager passes with HIP events around every attention call (the roofline)
    timer.on = True
    ms_eager = time_passes(torch, model, batch, caches, args.steps, attn_fn=attn, fused_head=True)
    timer.on = False
    # every call of one eager pass recorded by kernel class, each class then
    # replayed as a graph of its own calls (per-kernel rooflines and the
    # whole step's)
    with KernelCalls(torch) as kc:
        model.verify(batch, caches, fused_head=True)
    torch.cuda.synchronize()
    per_kernel, roof_ms_step = kernel_rooflines(env["sh"], N_REQ * K_CAND, ctx, kc.time_classes(), 1)
    # the timed step: the whole pass replayed as one HIP graph
    graph = model.capture(batch, caches, fused_head=True)
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    assert np.array_equal(batch.target.cpu().numpy(), tgt_bi), "graph replay changed targets"
    print(f"[bench] warmup done, timing {args.steps} graph replays", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        graph.replay()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = start.elapsed_time(end) / args.steps
    assert np.array_equal(batch.accept_len.cpu().numpy(), acc_bi), "graph replay changed decisions"
    gpu_state = gpu_state_under_load(torch, graph.replay)
    del graph
    W = N_REQ * K_CAND
    # the same pass with split-K GEMMs and load-adaptive attention splits
    # (not batch-invariant): slowdown = t_invariant / t_variant
    print("[bench] split-K / adaptive-split variant pass", file=sys.stderr, flush=True)
    from invariant_verify_verifier_amd.dvr import SplitKernels

    var = SplitKernels(N_REQ, env["sh"].kv_heads, env["lay"].max_blocks, tune=True)
    model.verify(batch, caches, attn_fn=var.attn, gemm_fn=var.gemm, fused_head=True)  # tunes each shape once
    torch.cuda.synchronize()
    # the invariant attention call, timed the way the variant's candidates were
    sh_ = env["sh"]
    a_q = torch.empty((N_REQ * K_CAND, sh_.heads * sh_.head_dim), dtype=torch.bfloat16, device="cuda").normal_()
    a_o = torch.empty((N_REQ * K_CAND, sh_.heads, sh_.head_dim), dtype=torch.bfloat16, device="cuda")
    t_attn_bi = _dvr_event_ms(lambda: biv.attn_decode_bi(a_q, caches[0][0], caches[0][1], batch.block_table, batch.ctx,
                                                         a_o, K_CAND, 1.0 / math.sqrt(sh_.head_dim),
                                                         model.workspace(N_REQ, env["lay"].max_blocks, K_CAND)))
    per_shape = {}
    for key, t in var.timings.items():
        if key[0] == "gemm":
            _, M_, N_, K_ = key
            best = var.splits[(M_, N_, K_)]
            per_shape[f"gemm M={M_} N={N_} K={K_}"] = {
                "us_by_splits": t, "chosen_splits": best,
                "t_invariant_us": t[1], "t_variant_us": t[best], "slowdown": round(t[1] / t[best], 4)}
        else:
            best = var.attn_splits[key[1:]]
            per_shape[f"attention R={key[1]} q_len={key[2]}"] = {
                "us_by_split_tokens": t, "chosen_split_tokens": best,
                "t_invariant_us": round(t_attn_bi * 1e3, 2), "t_variant_us": t[best],
                "slowdown": round(t_attn_bi * 1e3 / t[best], 4)}
    ms_var = time_graph(torch, model, batch, caches, args.steps, args.warmup, attn_fn=var.attn, gemm_fn=var.gemm,
                        fused_head=True)
    tgt_var = batch.target.cpu().numpy()
    acc_var = batch.accept_len.cpu().numpy()
    value = W / (ms_step / 1e3)
    sh = env["sh"]
    attn_bytes = float(np.sum(ctx.astype(np.int64) + K_CAND)) * sh.kv_heads * sh.head_dim * 2 * 2
    attn_ms = timer.mean_ms()
    achieved = attn_bytes / (attn_ms / 1e3) / 1e9
    line = {
        "metric": "verified tokens/s at W=N·K (1 GPU)",
        "value": round(value, 2),
        "unit": "verified tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "ms_per_step_eager": round(ms_eager, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded random-init weights and KV of the stated shapes)",
        "config": {"workload": f"Llama-3-8B-shaped verifier pass ({args.layers} layers, hidden 4096, 32/8 heads x 128, "
                               "FFN 14336, vocab 128256), W = N*K = 64*8 = 512, contexts U[2048,8192], "
                               "16-token pages, Gumbel verify + KV overwrite",
                   "N": N_REQ, "K": K_CAND, "W": W, "ctx_mean": float(ctx.mean()),
                   "launch": "whole pass captured as one HIP graph; lm_head + Gumbel verify fused",
                   "wall_s_timed": round(wall, 3)},
        "slowdown_vs_splitk": {"value": round(ms_step / ms_var, 4), "ms_variant": round(ms_var, 4),
                               "variant": "gemm_splitk and attn_decode_adaptive with the split of each shape "
                                          "chosen by timing the candidates (GEMM splits 1/2/4/8, 1 = the "
                                          "invariant kernel; KV splits 256*2^k tokens); same fused lm_head + "
                                          "Gumbel verify",
                               "per_shape": per_shape,
                               "target_rows_differing": int((tgt_var != tgt_bi).sum()),
                               "accept_len_differing": int((acc_var != acc_bi).sum())},
        "roofline": {"kernel": "attn_decode_bi (attn_bf16_kernel + attn_combine_kernel)", "bound": "hbm",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": recorded_traffic(),
                     "bytes_per_launch": attn_bytes, "avg_launch_ms": round(attn_ms, 5),
                     "launches_timed": len(timer.pairs)},
        "roofline_per_kernel": per_kernel,
        "roofline_step": {"roofline_ms": round(roof_ms_step, 4), "ms_per_step": round(ms_step, 4),
                          "frac": round(roof_ms_step / ms_step, 4),
                          "note": "sum over every call of the pass of max(algorithmic bytes / 8 TB/s, "
                                  "FLOP / 2.5 PFLOP/s bf16) at this run's contexts, divided by the timed step"},
        "cpu_baseline": None,
        "gpu_state": gpu_state,
    }
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle sample)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(torch, env, args.layers)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
