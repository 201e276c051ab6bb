"""CPU oracle for the batch-invariant verifier step — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, calls or links it, and shares no code with
it; the two meet only through the seeded inputs of ``workloads``.

Everything here is the plain definition of what the verifier computes, in
fp64 NumPy, with no blocking, fusion or reordering:

* the three batch-invariant kernels (post on batch-invariant computation and
  LLM-42, first paragraph: matmul, RMSNorm, attention) reach exactly the
  results of their plain definitions — fixing the reduction order changes only
  the rounding, never what is computed;
* the decoder forward over W = N*K candidate tokens (same post, third and
  fourth paragraphs: verifier forward at fixed batch, K tokens from each of N
  requests, overwrite of the fast path's KV);
* Gumbel-max verification (reading-club post on Gumbel coupling: add Gumbel
  noise, take the argmax, compare the draft token with the target token).

Every function is pinned by ``tests/test_oracle_*.py`` to something other than
itself (closed forms, brute force on tiny inputs, invariants, distributional
tests).  Functions without such a pin say "parity unpinned" in their docstring;
at present none does.
"""
from .ops import (  # noqa: F401
    as_f64,
    attention,
    decoder_forward,
    gumbel_sample,
    gumbel_topk,
    gumbel_verify,
    kv_copy_pages,
    kv_overwrite,
    linear,
    perturbed_scores,
    rmsnorm,
    rollback,
    rope,
    round_bf16,
    sequential_decode,
    silu,
    dvr_decode,
    tree_select,
    tree_verify,
)
