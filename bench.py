"""Benchmark: the batch-invariant verifier step on one MI355X.

One step = one verifier pass over W = N*K = 64*8 = 512 candidate tokens on a
Llama-3-8B-shaped decoder (32 layers, hidden 4096, 32 Q / 8 KV heads x 128,
SwiGLU FFN 14336, vocab 128256, RoPE theta 500000; bf16 random-init weights
N(0, 0.02)), contexts L_r ~ U[2048, 8192] in a paged KV cache of 16-token
pages, then Gumbel-max verification of the candidates (the KV overwrite of the
fast-path slots runs inside every layer).  Inputs are resident in HBM before
the timed region.

Prints ONE JSON line: verified tokens/s, the attention kernel's roofline
(HBM-bound; bytes = one read of each visible K/V row, timed with HIP events on
the stream it runs on), and the CPU oracle timed on a bounded sample.

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
    return p.parse_args()


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


def setup(torch, n_layers):
    import workloads as wl
    from invariant_verify_verifier_amd import verifier as V

    sh = wl.LLAMA3_8B
    ctx = wl.context_lengths(wl.SEEDS["pass_len"], N_REQ, CTX_LO, CTX_HI)
    lay = wl.paged_layout(ctx, K_CAND, seed=wl.SEEDS["pass_len"] + 1)
    dw = wl.device_model_weights(sh, wl.SEEDS["pass_weights"], layers=n_layers)
    caches = wl.device_kv_cache(sh, lay.num_blocks, wl.SEEDS["pass_kv"], layers=n_layers)
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
                noise=noise)


def cpu_baseline(torch, env, n_layers):
    """The oracle, untouched, on a bounded sample of the same workload: one
    decoder layer over all 512 rows plus the final norm, lm_head and verify,
    extrapolated to the full depth as 32 * t_layer + t_head per pass."""
    import oracle
    import workloads as wl
    from threadpoolctl import threadpool_info

    sh, dw, lay, ctx = env["sh"], env["dw"], env["lay"], env["ctx"]
    n = N_REQ
    H, D, F = sh.hidden, sh.head_dim, sh.ffn
    q, kv = sh.heads * D, sh.kv_heads * D

    def f64(t):
        b = t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)

    L0 = dw["layers"][0]
    wqkv, wgu = f64(L0["wqkv"]), f64(L0["w_gu"])
    layer = dict(attn_norm=f64(L0["attn_norm"]), wq=wqkv[:q], wk=wqkv[q:q + kv], wv=wqkv[q + kv:], wo=f64(L0["wo"]),
                 ffn_norm=f64(L0["ffn_norm"]), w_gate=wgu[:F], w_up=wgu[F:], w_down=f64(L0["w_down"]))
    ow = dict(shape=wl.ModelShape(1, H, sh.heads, sh.kv_heads, D, F, sh.vocab, sh.eps, sh.rope_theta),
              embed=f64(dw["embed"]), lm_head=None, final_norm=f64(dw["final_norm"]), layers=[layer])
    used = sorted({int(b) for b in lay.block_table[:n].ravel() if b >= 0})
    remap = {b: i for i, b in enumerate(used)}
    kc = f64(env["caches"][0][0][used])
    vc = f64(env["caches"][0][1][used])
    bt = np.vectorize(lambda b: remap.get(int(b), -1))(lay.block_table[:n]).astype(np.int32)
    toks = np.concatenate([env["t0"][:n, None], env["cand"][:n, :K_CAND - 1]], axis=1)
    lm = f64(dw["lm_head"])
    # one layer (the oracle's decoder forward with a 1-layer model and a
    # throwaway head), timed apart from the head
    ow["lm_head"] = lm[:1]
    t = time.perf_counter()
    oracle.decoder_forward(ow, toks, ctx[:n], [kc], [vc], bt)
    t_layer = time.perf_counter() - t
    x = wl.normal_f32(1, (n * K_CAND, H)).astype(np.float64)
    t = time.perf_counter()
    logits = oracle.linear(oracle.rmsnorm(x, ow["final_norm"], sh.eps), lm)
    oracle.gumbel_verify(logits.astype(np.float32).reshape(n, K_CAND, -1), env["noise"][:n], env["cand"][:n])
    t_head = time.perf_counter() - t
    t_pass = n_layers * t_layer + t_head
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": round(n * K_CAND / t_pass, 3), "unit": "verified tok/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"1 of {n_layers} layers + lm_head/verify over all {n * K_CAND} rows, fp64; "
                      f"t_layer={t_layer:.2f}s t_head={t_head:.2f}s; pass = {n_layers}*t_layer + t_head "
                      f"(extrapolated)"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only; --gpus {args.gpus} is not supported "
              "(the verifier step shards by request with no inter-GPU traffic; see the design notes)",
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
    print(f"[bench] warmup done, timing {args.steps} steps", file=sys.stderr, flush=True)
    timer.on = True
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        model.verify(batch, caches, attn_fn=attn)
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    timer.on = False
    ms_step = start.elapsed_time(end) / args.steps
    W = N_REQ * K_CAND
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
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded random-init weights and KV of the stated shapes)",
        "config": {"workload": f"Llama-3-8B-shaped verifier pass ({args.layers} layers, hidden 4096, 32/8 heads x 128, "
                               "FFN 14336, vocab 128256), W = N*K = 64*8 = 512, contexts U[2048,8192], "
                               "16-token pages, Gumbel verify + KV overwrite",
                   "N": N_REQ, "K": K_CAND, "W": W, "ctx_mean": float(ctx.mean()),
                   "wall_s_timed": round(wall, 3)},
        "roofline": {"kernel": "attn_bf16_kernel (attn_decode_bi)", "bound": "hbm",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "bytes_per_launch": attn_bytes, "avg_launch_ms": round(attn_ms, 5),
                     "launches_timed": len(timer.pairs)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle sample)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(torch, env, args.layers)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
