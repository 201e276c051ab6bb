"""Pins of the oracle's RMSNorm, matmul, RoPE, attention, KV overwrite and
bf16 rounding against closed forms, exact integer arithmetic, invariants and
brute-force loops on tiny inputs (never against a retyped copy of the same
vectorised formula)."""
import math

import numpy as np
import pytest

import oracle
import workloads as wl

# --------------------------------------------------------------------- RMSNorm


@pytest.mark.parametrize("c", [1e-3, 0.5, 3.0, -7.0])
def test_rmsnorm_constant_row_closed_form(c):
    """x = c*1 gives y = gamma * c / sqrt(c^2 + eps) (epsilon inside the root,
    mean over hidden)."""
    H, eps = 64, 1e-6
    gamma = np.linspace(0.5, 1.5, H)
    y = oracle.rmsnorm(np.full((1, H), c), gamma, eps)
    np.testing.assert_allclose(y[0], gamma * c / math.sqrt(c * c + eps), rtol=1e-14)


def test_rmsnorm_invariants():
    """gamma = 1: mean(y^2) = m / (m + eps) with m = mean(x^2); and with eps = 0
    the output is invariant to scaling x."""
    x = wl.normal_f32(1, (5, 300)).astype(np.float64) * 0.01
    eps = 1e-6
    y = oracle.rmsnorm(x, np.ones(300), eps)
    m = (x * x).mean(axis=1)
    np.testing.assert_allclose((y * y).mean(axis=1), m / (m + eps), rtol=1e-12)
    y0 = oracle.rmsnorm(x, np.ones(300), 0.0)
    np.testing.assert_allclose(oracle.rmsnorm(37.0 * x, np.ones(300), 0.0), y0, rtol=1e-13)


def test_rmsnorm_brute_force_loop():
    x = wl.normal_f32(2, (3, 7)).astype(np.float64)
    g = wl.normal_f32(3, (7,), 0.1, 1.0).astype(np.float64)
    y = oracle.rmsnorm(x, g, 1e-6)
    for i in range(3):
        ss = 0.0
        for k in range(7):
            ss += x[i, k] * x[i, k]
        r = math.sqrt(ss / 7 + 1e-6)
        for k in range(7):
            assert abs(y[i, k] - x[i, k] * g[k] / r) < 1e-13


# ---------------------------------------------------------------------- matmul


def test_linear_exact_integers_non_square():
    """Integer-valued operands: the fp64 product is exact; compare with Python
    integer arithmetic.  Non-square shapes catch a transposed operand."""
    g = wl.rng(4)
    a = g.integers(-3, 4, size=(3, 5))
    w = g.integers(-3, 4, size=(4, 5))  # [out, in]
    out = oracle.linear(a, w)
    assert out.shape == (3, 4)
    for m in range(3):
        for n in range(4):
            assert out[m, n] == sum(int(a[m, k]) * int(w[n, k]) for k in range(5))


# ------------------------------------------------------------------------ RoPE


def test_rope_hand_values():
    """D = 4, theta = 100: pair (0, 2) turns by pos rad, pair (1, 3) by
    pos * 100^(-1/2) = pos / 10 rad (rotate-half convention)."""
    x = np.array([[[1.0, 2.0, 0.0, 0.0]]])
    y = oracle.rope(x, np.array([3]), 100.0)[0, 0]
    np.testing.assert_allclose(y, [math.cos(3), 2 * math.cos(0.3), math.sin(3), 2 * math.sin(0.3)], rtol=1e-14)


def test_rope_invariants():
    """Position 0 is the identity; norms are preserved; q(m).k(n) depends only
    on m - n."""
    D = 128
    q = wl.normal_f32(5, (1, 1, D)).astype(np.float64)
    k = wl.normal_f32(6, (1, 1, D)).astype(np.float64)
    th = 500000.0
    np.testing.assert_array_equal(oracle.rope(q, [0], th), q)
    np.testing.assert_allclose(np.linalg.norm(oracle.rope(q, [777], th)), np.linalg.norm(q), rtol=1e-13)

    def dot(m, n):
        return float(oracle.rope(q, [m], th).ravel() @ oracle.rope(k, [n], th).ravel())

    assert abs(dot(10, 3) - dot(1007, 1000)) < 1e-9
    assert abs(dot(5000, 4000) - dot(1000, 0)) < 1e-9
    assert abs(dot(10, 3) - dot(10, 4)) > 1e-6


# ------------------------------------------------------------------- attention


def _contiguous_layout(ctx, q_len, block=16):
    need = [(int(c) + q_len + block - 1) // block for c in ctx]
    mb = max(need)
    bt = np.full((len(ctx), mb), -1, dtype=np.int32)
    o = 0
    for r, n in enumerate(need):
        bt[r, :n] = np.arange(o, o + n)
        o += n
    return bt, o


def test_attention_single_key_returns_v():
    """Row at position 0 sees one key: softmax weight 1, output = v exactly."""
    D = 8
    bt, nb = _contiguous_layout([0], 1)
    kc = wl.normal_f32(7, (nb, 1, 16, D)).astype(np.float64)
    vc = wl.normal_f32(8, (nb, 1, 16, D)).astype(np.float64)
    q = wl.normal_f32(9, (1, 1, D)).astype(np.float64)
    out = oracle.attention(q, kc, vc, bt, [0], 1, 0.3)
    np.testing.assert_array_equal(out[0, 0], vc[0, 0, 0])


def test_attention_zero_query_is_causal_mean_and_gqa_mapping():
    """q = 0: equal scores, output = mean of the visible V rows (positions
    0..ctx+j).  Four q heads over two KV heads: head h reads KV head h // 2."""
    D, Hq, Hkv, ctx, q_len = 4, 4, 2, 21, 3
    bt, nb = _contiguous_layout([ctx], q_len)
    kc = wl.normal_f32(10, (nb, Hkv, 16, D)).astype(np.float64)
    vc = wl.normal_f32(11, (nb, Hkv, 16, D)).astype(np.float64)
    q = np.zeros((q_len, Hq, D))
    out = oracle.attention(q, kc, vc, bt, [ctx], q_len, 1.0)
    flat = vc.transpose(1, 0, 2, 3).reshape(Hkv, -1, D)  # contiguous pages -> positions
    for j in range(q_len):
        for h in range(Hq):
            np.testing.assert_allclose(out[j, h], flat[h // 2, : ctx + j + 1].mean(axis=0), rtol=1e-12, atol=1e-14)


def test_attention_masked_keys_do_not_matter_and_pages_permute():
    """Keys after a row's position do not change its output (NaN there is
    fine); permuting the physical pages does not change anything."""
    D, Hq, Hkv, q_len = 8, 2, 1, 4
    ctx = [37, 5]
    lay = wl.paged_layout(ctx, q_len, seed=3, spare_blocks=2)
    kc = wl.normal_f32(12, (lay.num_blocks, Hkv, 16, D)).astype(np.float64)
    vc = wl.normal_f32(13, (lay.num_blocks, Hkv, 16, D)).astype(np.float64)
    q = wl.normal_f32(14, (2 * q_len, Hq, D)).astype(np.float64)
    out = oracle.attention(q, kc, vc, lay.block_table, ctx, q_len, 0.35)
    # poison every position > ctx[r] (row j = 0 must not see them)
    kc2, vc2 = kc.copy(), vc.copy()
    for r in range(2):
        for p in range(ctx[r] + 1, lay.max_blocks * 16):
            b = lay.block_table[r, p // 16]
            if b >= 0:
                kc2[b, :, p % 16] = np.nan
                vc2[b, :, p % 16] = np.nan
    out2 = oracle.attention(q.reshape(2, q_len, Hq, D)[:, :1].reshape(2, Hq, D), kc2, vc2,
                            lay.block_table, ctx, 1, 0.35)
    np.testing.assert_array_equal(out2, out.reshape(2, q_len, Hq, D)[:, 0])
    # contiguous pages
    bt, nb = _contiguous_layout(ctx, q_len)
    kc3 = np.zeros((nb, Hkv, 16, D))
    vc3 = np.zeros((nb, Hkv, 16, D))
    for r in range(2):
        for b in range(lay.max_blocks):
            if lay.block_table[r, b] >= 0 and bt[r, b] >= 0:
                kc3[bt[r, b]] = kc[lay.block_table[r, b]]
                vc3[bt[r, b]] = vc[lay.block_table[r, b]]
    np.testing.assert_allclose(oracle.attention(q, kc3, vc3, bt, ctx, q_len, 0.35), out, rtol=1e-13)


def test_attention_brute_force_loop():
    """Scalar-loop softmax attention on a tiny case."""
    D, Hq, Hkv, q_len, ctx = 3, 2, 1, 2, [4]
    bt, nb = _contiguous_layout(ctx, q_len)
    kc = wl.normal_f32(15, (nb, Hkv, 16, D)).astype(np.float64)
    vc = wl.normal_f32(16, (nb, Hkv, 16, D)).astype(np.float64)
    q = wl.normal_f32(17, (q_len, Hq, D)).astype(np.float64)
    out = oracle.attention(q, kc, vc, bt, ctx, q_len, 0.5)
    for j in range(q_len):
        for h in range(Hq):
            n = ctx[0] + j + 1
            sc = [0.5 * sum(q[j, h, d] * kc[0, 0, p, d] for d in range(D)) for p in range(n)]
            mx = max(sc)
            ex = [math.exp(s - mx) for s in sc]
            tot = sum(ex)
            for d in range(D):
                ref = sum(ex[p] / tot * vc[0, 0, p, d] for p in range(n))
                assert abs(out[j, h, d] - ref) < 1e-13


def test_attention_dominant_key():
    """One key aligned with a large query dominates: output ~ its v."""
    D = 16
    bt, nb = _contiguous_layout([40], 1)
    kc = wl.normal_f32(18, (nb, 1, 16, D)).astype(np.float64) * 0.01
    vc = wl.normal_f32(19, (nb, 1, 16, D)).astype(np.float64)
    kc[1, 0, 7] = 1.0  # position 23
    q = np.full((1, 1, D), 1.0)
    out = oracle.attention(q, kc, vc, bt, [40], 1, 10.0)
    np.testing.assert_allclose(out[0, 0], vc[1, 0, 7], rtol=1e-9, atol=1e-9)


# --------------------------------------------------------------- KV overwrite


def test_kv_overwrite_exact_and_local():
    kc = np.full((3, 2, 16, 4), 5.0)
    vc = np.full((3, 2, 16, 4), -5.0)
    kn = wl.normal_f32(20, (2, 2, 4)).astype(np.float64)
    vn = wl.normal_f32(21, (2, 2, 4)).astype(np.float64)
    oracle.kv_overwrite(kc, vc, kn, vn, [17, 40])
    np.testing.assert_array_equal(kc[1, :, 1], kn[0])
    np.testing.assert_array_equal(vc[2, :, 8], vn[1])
    mask = np.ones(kc.shape, dtype=bool)
    mask[1, :, 1] = False
    mask[2, :, 8] = False
    assert (kc[mask] == 5.0).all() and (vc[mask] == -5.0).all()


# -------------------------------------------------------------- bf16 rounding


def test_round_bf16_matches_bit_level_rne_on_fp32_values():
    """For values that are exactly fp32, rounding once to bf16 must agree with
    the bit-level RNE of the input generator (an independent implementation),
    including the exact-tie cases."""
    x = np.concatenate([wl.normal_f32(22, (20000,), 5.0),
                        np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 2 ** -100, 3e38 / 2],
                                 dtype=np.float32)])
    ref = wl.bf16_to_f32(wl.bf16_bits(x)).astype(np.float64)
    np.testing.assert_array_equal(oracle.round_bf16(x.astype(np.float64)), ref)
    assert oracle.round_bf16(np.array([1 + 2 ** -8]))[0] == 1.0       # tie to even (down)
    assert oracle.round_bf16(np.array([1 + 3 * 2 ** -8]))[0] == 1 + 2 ** -6  # tie to even (up)


def test_silu_closed_forms():
    """silu(z) = z * sigmoid(z), pinned by values fixed by the mathematics:
    silu(0) = 0; sigmoid(ln 3) = 3/4 and sigmoid(-ln 3) = 1/4, so
    silu(+-ln 3) = +-(3/4, 1/4) ln 3; silu(z) - silu(-z) = z for every z;
    silu(z) -> z for large z and -> 0 for very negative z.  A dropped sign,
    a missing factor z or sigmoid(-z) in place of sigmoid(z) fails one."""
    ln3 = math.log(3.0)
    got = oracle.silu(np.array([0.0, ln3, -ln3, 40.0, -40.0]))
    assert got[0] == 0.0
    assert abs(got[1] - 0.75 * ln3) < 1e-15 and abs(got[2] + 0.25 * ln3) < 1e-15
    assert abs(got[3] - 40.0) < 1e-12 and abs(got[4]) < 1e-15
    z = np.linspace(-9.0, 9.0, 181)
    np.testing.assert_allclose(oracle.silu(z) - oracle.silu(-z), z, rtol=0, atol=1e-13)
