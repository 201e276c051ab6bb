"""GPU parity of each kernel against the CPU oracle, and batch invariance of
the "_bi" kernels checked bitwise on the GPU itself.

Parity: bit-exact for gumbel_verify and kv_overwrite (integer/byte work and an
argmax taken in the same fp32 precision on both sides); tolerances from
tests/tolerances.py for floating point.  Invariance (LLM-42 post, paragraph 1:
the same result whatever the batch size): a row's output bits must not change
with M, with its position in the batch or with the rows next to it.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_util import DEV, announce, bits, dev_bf16, dev_f32, dev_i32, dev_i64, f64, sync
from tolerances import bf16_step, check_bf16, check_f32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def biv():
    import invariant_verify_verifier_amd as m

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


# =====================================================================
# gumbel_verify
# =====================================================================


def _plant_ties(logits, noise, frac_near, frac_exact, seed):
    """Plant near-ties (0 < top-2 gap of s < 1e-3) and exact fp32 ties in the
    perturbed scores s = fl32(l + g) of some rows, on either side of the max."""
    g = wl.rng(seed)
    R, K, V = logits.shape
    s = oracle.perturbed_scores(logits, noise)
    rows = [(r, j) for r in range(R) for j in range(K)]
    n_near = int(round(frac_near * len(rows)))
    n_exact = int(round(frac_exact * len(rows)))
    pick = g.permutation(len(rows))
    planted_exact = 0
    for k, idx in enumerate(pick[:n_near]):
        r, j = rows[idx]
        t = int(np.argmax(s[r, j]))
        u = int(g.integers(0, V - 1))
        u = u + (u >= t)
        want = np.float32(s[r, j, t])
        if k < n_exact:
            lu = np.float32(want - noise[r, j, u])
            for _ in range(64):
                got = np.float32(lu + noise[r, j, u])
                if got == want:
                    break
                lu = np.nextafter(lu, np.float32(np.inf) if got < want else np.float32(-np.inf), dtype=np.float32)
            if np.float32(lu + noise[r, j, u]) == want:
                logits[r, j, u] = lu
                planted_exact += 1
        else:
            delta = np.float32(g.uniform(1e-5, 1e-3))
            logits[r, j, u] = np.float32(want - delta - noise[r, j, u])
    return planted_exact


def _verify_case(biv, R, K, V, seed, near=0.05, exact=0.01, offset=0):
    logits = wl.normal_f32(seed, (R, K, V), std=3.0)
    noise = wl.gumbel_noise(seed + 3, np.repeat(np.arange(R), K), np.tile(np.arange(K) + 5000, R), V).reshape(R, K, V)
    n_exact = _plant_ties(logits, noise, near, exact, seed + 1)
    t0, _, _ = oracle.gumbel_verify(logits, noise, np.zeros((R, K), np.int32))
    d = wl.rng(seed + 2).integers(0, K + 1, size=R)
    cand = wl.plant_divergence(t0, d, V, seed + 2)
    t_ref, a_ref, n_ref = oracle.gumbel_verify(logits, noise, cand)
    assert np.array_equal(a_ref, d)
    if offset:  # misaligned rows: exercise the scalar path
        lg = torch.zeros(R * K * V + offset, dtype=torch.float32, device=DEV)
        nz = torch.zeros_like(lg)
        lg[offset:] = dev_f32(logits.reshape(-1))
        nz[offset:] = dev_f32(noise.reshape(-1))
        lg, nz = lg[offset:].view(R * K, V), nz[offset:].view(R * K, V)
    else:
        lg, nz = dev_f32(logits.reshape(R * K, V)), dev_f32(noise.reshape(R * K, V))
    c = dev_i32(cand)
    tgt = torch.full((R, K), -7, dtype=torch.int32, device=DEV)
    acc = torch.full((R,), -7, dtype=torch.int32, device=DEV)
    nxt = torch.full((R,), -7, dtype=torch.int32, device=DEV)
    announce("gumbel_verify", R, K, V, seed, offset)
    biv.gumbel_verify(lg, nz, c, tgt, acc, nxt)
    sync()
    assert np.array_equal(tgt.cpu().numpy(), t_ref)
    assert np.array_equal(acc.cpu().numpy(), a_ref)
    assert np.array_equal(nxt.cpu().numpy(), n_ref)
    return n_exact


def test_gumbel_verify_full_size_bitwise(biv):
    """Full-size coupled verify: fp32 logits [64, 8, 128256] ~ N(0, 9), near-ties
    in 5% of rows (1% exact), first divergence d ~ U{0..8}."""
    n_exact = _verify_case(biv, 64, 8, 128256, seed=30)
    assert n_exact >= 3


@pytest.mark.parametrize("R,K,V,offset", [(3, 4, 4099, 0), (2, 3, 1000, 1), (5, 1, 257, 0), (1, 8, 2, 0),
                                          (16, 4, 4096, 0)])
def test_gumbel_verify_edge_shapes_bitwise(biv, R, K, V, offset):
    _verify_case(biv, R, K, V, seed=40 + V % 7, near=0.5, exact=0.25, offset=offset)


def test_gumbel_verify_nan_inf_rows(biv):
    V = 1000
    l = wl.normal_f32(5, (2, 3, V))
    g = np.zeros((2, 3, V), np.float32)
    l[0, 0, :] = np.nan
    l[0, 1, ::2] = np.nan
    l[0, 2, :] = -np.inf
    l[1, 0, 17] = np.inf
    l[1, 1, 5] = np.float32(-0.0)
    l[1, 1, :] = np.float32(-1.0)
    l[1, 1, 5] = np.float32(-0.0)
    l[1, 1, 3] = np.float32(0.0)
    cand = np.zeros((2, 3), np.int32)
    t_ref, a_ref, n_ref = oracle.gumbel_verify(l, g, cand)
    tgt = torch.empty((2, 3), dtype=torch.int32, device=DEV)
    acc = torch.empty(2, dtype=torch.int32, device=DEV)
    nxt = torch.empty(2, dtype=torch.int32, device=DEV)
    announce("gumbel_verify nan/inf")
    biv.gumbel_verify(dev_f32(l.reshape(6, V)), dev_f32(g.reshape(6, V)), dev_i32(cand), tgt, acc, nxt)
    sync()
    assert np.array_equal(tgt.cpu().numpy(), t_ref)
    assert t_ref[0, 0] == 0 and t_ref[1, 1] == 3 and t_ref[1, 0] == 17
    assert np.array_equal(acc.cpu().numpy(), a_ref) and np.array_equal(nxt.cpu().numpy(), n_ref)


@pytest.mark.parametrize("rows,V,k", [(512, 128256, 8), (7, 1001, 3), (3, 5, 5), (40, 4096, 1)])
def test_gumbel_topk_bitwise(biv, rows, V, k):
    """Indices and scores bit for bit the oracle's, with planted exact ties, NaN
    and -inf entries, and an all-NaN row; k = 1 equals gumbel_verify's target."""
    l = wl.normal_f32(140 + V % 11, (rows, V), std=3.0)
    g = wl.gumbel_noise(141, np.arange(rows), np.full(rows, 500), V)
    if V > 20:
        l[0, [3, 11, 17]] = np.float32(1e9)  # three-way exact tie
        l[1, ::5] = np.nan
        l[2 % rows, 1::2] = -np.inf
    l[rows - 1, :] = np.nan
    i_ref, s_ref = oracle.gumbel_topk(l, g, k)
    idx = torch.full((rows, k), -3, dtype=torch.int32, device=DEV)
    sc = torch.full((rows, k), 7.0, dtype=torch.float32, device=DEV)
    announce("gumbel_topk", rows, V, k)
    biv.gumbel_topk(dev_f32(l), dev_f32(g), idx, sc)
    sync()
    assert np.array_equal(idx.cpu().numpy(), i_ref)
    assert np.array_equal(sc.cpu().numpy().view(np.uint32), s_ref.astype(np.float32).view(np.uint32))
    if V > 20:
        assert list(i_ref[0, :min(k, 3)]) == [3, 11, 17][:min(k, 3)]
    if k == 1:
        t_ref, _, _ = oracle.gumbel_verify(l[:, None, :], g[:, None, :], np.zeros((rows, 1), np.int32))
        assert np.array_equal(i_ref[:, 0], t_ref[:, 0])


# =====================================================================
# lm_head_gumbel_verify (lm_head matmul with the Gumbel argmax in its epilogue)
# =====================================================================


@pytest.mark.parametrize("R,K,V", [(5, 8, 128256), (3, 3, 50021), (12, 8, 50021)])
def test_lm_head_gumbel_verify_bitwise(biv, R, K, V):
    """The fused call gives the bits of gemm_bi (fp32 logits) + gumbel_verify,
    and both equal the oracle's rule applied to the GPU's logits.  Planted in
    the noise: an exact tie at 1e9 between two columns in different 256-column
    tiles (the lower index must win), NaNs at a row's best entries, an
    all-NaN row (target 0), and -inf entries.  V = 50021 leaves a ragged last
    tile and group; M = R*K rows leave a ragged last row tile."""
    H = 4096
    M = R * K
    h = dev_bf16(wl.normal_bf16(120 + V % 5, (M, H)))
    w = dev_bf16(wl.normal_bf16(121, (V, H), std=0.02))
    logits = torch.empty((M, V), dtype=torch.float32, device=DEV)
    announce("lm_head_gumbel_verify: unfused logits", R, K, V)
    biv.gemm_bi(h, w, logits)
    sync()
    l32 = logits.cpu().numpy()
    g = wl.gumbel_noise(122, np.repeat(np.arange(R), K).reshape(R, K),
                        np.tile(np.arange(K) + 300, (R, 1)), V).reshape(M, V)
    c1, c2 = 77, V - 200  # different 256-column tiles and 64-column groups
    g[3, c1] = g[3, c2] = np.float32(1e9)  # |logit| << ulp(1e9) / 2: both scores are exactly 1e9
    best = np.argsort(l32[5] + g[5])[-3:]
    g[5, best] = np.nan  # the row's three best entries can never win
    g[min(7, M - 1), :] = np.nan  # all-NaN row: target 0
    g[1, ::3] = -np.inf
    s_ref, _, _ = oracle.gumbel_verify(l32.reshape(R, K, V), g.reshape(R, K, V), np.zeros((R, K), np.int32))
    assert s_ref[3 // K, 3 % K] == c1 and s_ref[min(7, M - 1) // K, min(7, M - 1) % K] == 0
    d = wl.rng(123).integers(0, K + 1, size=R)
    cand = wl.plant_divergence(s_ref, d, V, 124)
    t_ref, a_ref, n_ref = oracle.gumbel_verify(l32.reshape(R, K, V), g.reshape(R, K, V), cand)
    assert np.array_equal(a_ref, d)
    outs = []
    for fused in (False, True):
        tgt = torch.full((R, K), -5, dtype=torch.int32, device=DEV)
        acc = torch.full((R,), -5, dtype=torch.int32, device=DEV)
        nxt = torch.full((R,), -5, dtype=torch.int32, device=DEV)
        gd = dev_f32(g)
        announce("lm_head_gumbel_verify fused" if fused else "gumbel_verify on the logits", R, K, V)
        if fused:
            ws = torch.empty(biv.gumbel_workspace_bytes(M, V), dtype=torch.uint8, device=DEV)
            biv.lm_head_gumbel_verify(h, w, gd, dev_i32(cand), tgt, acc, nxt, ws)
        else:
            biv.gumbel_verify(logits, gd, dev_i32(cand), tgt, acc, nxt)
        sync()
        outs.append((tgt.cpu().numpy(), acc.cpu().numpy(), nxt.cpu().numpy()))
    for got in outs:
        assert np.array_equal(got[0], t_ref) and np.array_equal(got[1], a_ref) and np.array_equal(got[2], n_ref)


# =====================================================================
# kv_overwrite
# =====================================================================


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_kv_overwrite_bitwise(biv, dtype):
    """Only the named slots change, to the exact source bits; slots outside
    the cache are skipped; the source may be a strided slice of a fused row."""
    nb, Hkv, D, T = 37, 8, 128, 50
    g = wl.rng(3)
    slots = g.permutation(nb * 16)[:T].astype(np.int64)
    slots[7] = -1
    slots[13] = nb * 16 + 5
    width = 3 * Hkv * D
    if dtype == "bf16":
        src_np = wl.normal_bf16(4, (T, width))
        kc_np = wl.normal_bf16(5, (nb, Hkv, 16, D))
        vc_np = wl.normal_bf16(6, (nb, Hkv, 16, D))
        src, kc, vc = dev_bf16(src_np), dev_bf16(kc_np), dev_bf16(vc_np)
    else:
        src_np = wl.normal_f32(4, (T, width))
        kc_np = wl.normal_f32(5, (nb, Hkv, 16, D))
        vc_np = wl.normal_f32(6, (nb, Hkv, 16, D))
        src, kc, vc = dev_f32(src_np), dev_f32(kc_np), dev_f32(vc_np)
    kref, vref = kc_np.copy(), vc_np.copy()
    kn = src_np[:, Hkv * D:2 * Hkv * D].reshape(T, Hkv, D)
    vn = src_np[:, 2 * Hkv * D:].reshape(T, Hkv, D)
    ok = (slots >= 0) & (slots < nb * 16)
    oracle.kv_overwrite(kref, vref, kn[ok], vn[ok], slots[ok])
    announce("kv_overwrite", dtype)
    biv.kv_overwrite(src[:, Hkv * D:2 * Hkv * D], src[:, 2 * Hkv * D:], dev_i64(slots), kc, vc)
    sync()
    assert np.array_equal(bits(kc), kref.view(bits(kc).dtype))
    assert np.array_equal(bits(vc), vref.view(bits(vc).dtype))


@pytest.mark.parametrize("dtype,extra_cols", [("bf16", 0), ("bf16", 8), ("bf16", 3), ("f32", 0)])
def test_rope_kv_overwrite_matches_the_two_calls(biv, dtype, extra_cols):
    """The fused RoPE + KV overwrite gives the bits of rope_apply followed by
    kv_overwrite (Q and K rotated in the row, rotated K and raw V in the
    cache), and both match the oracle; rows with a position outside the table
    stay unrotated, slots outside the cache are skipped.  extra_cols pads the
    row stride (3 makes bf16 rows unaligned, which takes the two-call path)."""
    nb, Hq, Hkv, D, T = 41, 32, 8, 128, 67
    width = (Hq + 2 * Hkv) * D + extra_cols
    g = wl.rng(21)
    slots = g.permutation(nb * 16)[:T].astype(np.int64)
    slots[5], slots[60] = -3, nb * 16
    pos = g.integers(0, 4096, size=T).astype(np.int32)
    pos[9], pos[11] = -1, 4096
    dev, mk = (dev_bf16, wl.normal_bf16) if dtype == "bf16" else (dev_f32, wl.normal_f32)
    src_np = mk(22, (T, width))
    kc_np, vc_np = mk(23, (nb, Hkv, 16, D)), mk(24, (nb, Hkv, 16, D))
    table = biv.rope_table(4096, D, 500000.0).to(DEV)
    x1, k1, v1 = dev(src_np), dev(kc_np), dev(vc_np)
    x2, k2, v2 = dev(src_np), dev(kc_np), dev(vc_np)
    ps, sl = dev_i32(pos), dev_i64(slots)
    announce("rope_kv_overwrite", dtype, extra_cols)
    biv.rope_kv_overwrite(x1, ps, table, sl, k1, v1, Hq)
    biv.rope_apply(x2, ps, table, Hq + Hkv, D)
    biv.kv_overwrite(x2[:, Hq * D:(Hq + Hkv) * D], x2[:, (Hq + Hkv) * D:(Hq + 2 * Hkv) * D], sl, k2, v2)
    sync()
    for a, b, what in [(x1, x2, "rows"), (k1, k2, "k cache"), (v1, v2, "v cache")]:
        assert np.array_equal(bits(a), bits(b)), what
    # oracle: rotate the rows in fp64, then overwrite the valid slots
    ref = oracle.as_f64(src_np, dtype).copy()
    ok_pos = (pos >= 0) & (pos < 4096)
    rot = ref[ok_pos, :(Hq + Hkv) * D].reshape(-1, Hq + Hkv, D)
    ref[ok_pos, :(Hq + Hkv) * D] = oracle.rope(rot, pos[ok_pos], 500000.0).reshape(-1, (Hq + Hkv) * D)
    chk = (lambda g_, r, w: check_bf16(g_, r, w)) if dtype == "bf16" else (lambda g_, r, w: check_f32(g_, r, what=w))
    chk(f64(x1), ref, "rotated rows")
    ok = (slots >= 0) & (slots < nb * 16)
    kref = oracle.as_f64(kc_np, dtype).copy()
    vref = oracle.as_f64(vc_np, dtype).copy()
    kn = f64(x1)[:, Hq * D:(Hq + Hkv) * D].reshape(T, Hkv, D)
    vn = oracle.as_f64(src_np, dtype)[:, (Hq + Hkv) * D:(Hq + 2 * Hkv) * D].reshape(T, Hkv, D)
    oracle.kv_overwrite(kref, vref, kn[ok], vn[ok], slots[ok])
    assert np.array_equal(f64(k1), kref) and np.array_equal(f64(v1), vref)


# =====================================================================
# rmsnorm_bi
# =====================================================================

M_SWEEP = [1, 2, 4, 8, 16, 32, 64, 128, 256, 512]


def test_rmsnorm_bf16_parity_and_invariance(biv):
    """bf16 activations [M, 4096] ~ N(0,1), gamma ~ N(1, 0.1), eps 1e-6."""
    H = 4096
    x_np = wl.normal_bf16(10, (512, H))
    g_np = wl.normal_bf16(11, (H,), std=0.1, mean=1.0)
    x, gam = dev_bf16(x_np), dev_bf16(g_np)
    announce("rmsnorm bf16 M=512")
    y = torch.empty_like(x)
    biv.rmsnorm_bi(x, gam, y, 1e-6)
    sync()
    ref = oracle.rmsnorm(oracle.as_f64(x_np, "bf16"), oracle.as_f64(g_np, "bf16"), 1e-6)
    check_bf16(f64(y), ref, "rmsnorm bf16")
    full = bits(y)
    for M in M_SWEEP:
        yM = torch.empty((M, H), dtype=torch.bfloat16, device=DEV)
        biv.rmsnorm_bi(x[:M].contiguous(), gam, yM, 1e-6)
        sync()
        assert np.array_equal(bits(yM), full[:M]), f"rows changed at M={M}"
    perm = wl.rng(1).permutation(512)
    yp = torch.empty_like(x)
    biv.rmsnorm_bi(x[torch.from_numpy(perm).to(DEV)].contiguous(), gam, yp, 1e-6)
    sync()
    assert np.array_equal(bits(yp), full[perm])


def test_rmsnorm_f32_and_mixed(biv):
    H = 256
    x_np = wl.normal_f32(12, (37, H), std=2.0)
    g_np = wl.normal_f32(13, (H,), std=0.1, mean=1.0)
    ref = oracle.rmsnorm(x_np.astype(np.float64), g_np.astype(np.float64), 1e-6)
    y = torch.empty((37, H), dtype=torch.float32, device=DEV)
    announce("rmsnorm f32")
    biv.rmsnorm_bi(dev_f32(x_np), dev_f32(g_np), y, 1e-6)
    sync()
    check_f32(f64(y), ref, what="rmsnorm f32")
    # fp32 residual stream -> bf16 normalised activations
    gb = wl.bf16_bits(g_np)
    ref2 = oracle.rmsnorm(x_np.astype(np.float64), oracle.as_f64(gb, "bf16"), 1e-6)
    y2 = torch.empty((37, H), dtype=torch.bfloat16, device=DEV)
    biv.rmsnorm_bi(dev_f32(x_np), dev_bf16(gb), y2, 1e-6)
    sync()
    check_bf16(f64(y2), ref2, "rmsnorm f32->bf16")


@pytest.mark.parametrize("H", [1024, 4096, 8192])
def test_rmsnorm_vector_path_f32_residual(biv, H):
    """The decoder's call: an fp32 residual stream normalised into bf16 (and
    into fp32) through the 4-element vector path, on a ragged row count, with
    row bits independent of M; a 16-byte-misaligned input takes the scalar
    path and stays within the same bound."""
    Mx = 300
    x_np = wl.normal_f32(14 + H, (Mx, H), std=2.0)
    g_np = wl.normal_f32(15 + H, (H,), std=0.1, mean=1.0)
    gb = wl.bf16_bits(g_np)
    x = dev_f32(x_np)
    announce("rmsnorm vector path", H)
    y = torch.empty((Mx, H), dtype=torch.bfloat16, device=DEV)
    biv.rmsnorm_bi(x, dev_bf16(gb), y, 1e-6)
    yf = torch.empty((Mx, H), dtype=torch.float32, device=DEV)
    biv.rmsnorm_bi(x, dev_f32(g_np), yf, 1e-6)
    sync()
    check_bf16(f64(y), oracle.rmsnorm(x_np.astype(np.float64), oracle.as_f64(gb, "bf16"), 1e-6), "rmsnorm vec bf16")
    check_f32(f64(yf), oracle.rmsnorm(x_np.astype(np.float64), g_np.astype(np.float64), 1e-6), axis=1,
              what="rmsnorm vec f32")
    full = bits(y)
    for M in (1, 7, 64, 299):
        yM = torch.empty((M, H), dtype=torch.bfloat16, device=DEV)
        biv.rmsnorm_bi(x[:M].contiguous(), dev_bf16(gb), yM, 1e-6)
        sync()
        assert np.array_equal(bits(yM), full[:M]), f"rows changed at M={M}"
    # misaligned rows (offset by one element) -> the scalar kernel, which owns
    # and adds the same elements in the same order: the same bits
    buf = torch.empty(Mx * H + 1, dtype=torch.float32, device=DEV)
    xm = buf[1:].view(Mx, H)
    xm.copy_(x)
    ym = torch.empty(Mx * H + 1, dtype=torch.bfloat16, device=DEV)[1:].view(Mx, H)
    biv.rmsnorm_bi(xm, dev_bf16(gb), ym, 1e-6)
    sync()
    check_bf16(f64(ym), oracle.rmsnorm(x_np.astype(np.float64), oracle.as_f64(gb, "bf16"), 1e-6), "rmsnorm misaligned")
    assert np.array_equal(bits(ym), full), "misaligned x and y changed the bits"
    # only the output misaligned, or only gamma: the same bits again
    yo = torch.empty(Mx * H + 1, dtype=torch.bfloat16, device=DEV)[1:].view(Mx, H)
    biv.rmsnorm_bi(x, dev_bf16(gb), yo, 1e-6)
    gm = torch.empty(H + 1, dtype=torch.bfloat16, device=DEV)[1:]
    gm.copy_(dev_bf16(gb))
    yg = torch.empty((Mx, H), dtype=torch.bfloat16, device=DEV)
    biv.rmsnorm_bi(x, gm, yg, 1e-6)
    sync()
    assert np.array_equal(bits(yo), full), "a misaligned output changed the bits"
    assert np.array_equal(bits(yg), full), "a misaligned gamma changed the bits"


@pytest.mark.parametrize("dt,H,M", [("bf16", 4096, 300), ("f32", 4096, 37), ("bf16", 1000, 19), ("f32", 2048, 5)])
def test_rmsnorm_fused_residual(biv, dt, H, M):
    """rmsnorm_bi with a residual: s = x + residual stored back (rounded once to
    the activation dtype), y = rmsnorm(s).  Against the oracle: s is the exact
    sum rounded once (within one rounding of it), y is the fp64 norm of the
    stored s; bitwise equal to adding first and normalising s alone, and row
    bits independent of M and of the vector/scalar kernel."""
    if dt == "bf16":
        xb, rb = wl.normal_bf16(60 + H, (M, H)), wl.normal_bf16(61 + H, (M, H), std=3.0)
        x64, r64 = oracle.as_f64(xb, "bf16"), oracle.as_f64(rb, "bf16")
        x, r = dev_bf16(xb), dev_bf16(rb)
        s_ref = oracle.round_bf16(x64 + r64)
    else:
        xf, rf = wl.normal_f32(60 + H, (M, H)), wl.normal_f32(61 + H, (M, H), std=3.0)
        x64, r64 = xf.astype(np.float64), rf.astype(np.float64)
        x, r = dev_f32(xf), dev_f32(rf)
        s_ref = (x64 + r64).astype(np.float32).astype(np.float64)
    gb = wl.normal_bf16(62 + H, (H,), std=0.1, mean=1.0)
    g64 = oracle.as_f64(gb, "bf16")
    gam = dev_bf16(gb)
    announce("rmsnorm fused residual", dt, H, M)
    res = r.clone()
    y = torch.empty((M, H), dtype=torch.bfloat16, device=DEV)
    biv.rmsnorm_bi(x, gam, y, 1e-6, residual=res)
    sync()
    s_gpu = f64(res)
    if dt == "bf16":  # one fp32 add of two bf16 values, then one rounding to bf16: at most one step apart
        assert np.all(np.abs(s_gpu - s_ref) <= bf16_step(s_ref))
        assert np.mean(s_gpu == s_ref) > 0.9999
    else:
        assert np.array_equal(s_gpu, s_ref), "fp32 residual add is one IEEE add"
    check_bf16(f64(y), oracle.rmsnorm(s_gpu, g64, 1e-6), "rmsnorm of the stored residual")
    check_bf16(f64(y), oracle.rmsnorm(x64 + r64, g64, 1e-6), "rmsnorm of the exact sum")
    # fused == add, then normalise the stored sum with no residual
    y2 = torch.empty_like(y)
    biv.rmsnorm_bi(res.clone(), gam, y2, 1e-6)
    sync()
    assert np.array_equal(bits(y2), bits(y))
    # M-invariance of the fused call
    full = bits(y)
    for m in (1, M // 2 + 1):
        rm = r[:m].clone()
        ym = torch.empty((m, H), dtype=torch.bfloat16, device=DEV)
        biv.rmsnorm_bi(x[:m].contiguous(), gam, ym, 1e-6, residual=rm)
        sync()
        assert np.array_equal(bits(ym), full[:m]) and np.array_equal(bits(rm), bits(res)[:m])



# =====================================================================
# gemm_bi
# =====================================================================


def test_gemm_bf16_exact_integer_operands(biv):
    """Integer operands in {-2..2}: every partial sum is an exact fp32 integer
    (|sum| <= 4*4096 < 2^24), so any correct reduction equals the exact
    product -- the GPU must match the oracle bit for bit (fp32 output)."""
    M, N, K = 100, 300, 4096
    g = wl.rng(7)
    a = g.integers(-2, 3, size=(M, K)).astype(np.float32)
    b = g.integers(-2, 3, size=(N, K)).astype(np.float32)
    c = torch.empty((M, N), dtype=torch.float32, device=DEV)
    announce("gemm bf16 exact ints")
    biv.gemm_bi(dev_bf16(wl.bf16_bits(a)), dev_bf16(wl.bf16_bits(b)), c)
    sync()
    assert np.array_equal(c.cpu().numpy().astype(np.float64), oracle.linear(a, b))


def _microbench_weight(N=14336, K=4096):
    """The microbench weight is [4096, 14336] ~ N(0, 0.02); the GEMM takes it in
    linear-layer layout [N, K] (a one-time transpose, off the timed path)."""
    w = wl.normal_bf16(12, (K, N), std=0.02)
    return np.ascontiguousarray(w.T)


def test_gemm_bf16_14336x4096_microbench_parity_and_invariance(biv):
    """[M, 4096] x [4096, 14336], bf16 in, fp32 accumulate; every row's bits
    identical for M = 1, 2, 4, ..., 512 and under a row shuffle."""
    K, N = 4096, 14336
    a_np = wl.normal_bf16(10, (512, K))
    w_np = _microbench_weight(N, K)
    a, w = dev_bf16(a_np), dev_bf16(w_np)
    announce("gemm bf16 14336x4096 M=512")
    c = torch.empty((512, N), dtype=torch.bfloat16, device=DEV)
    biv.gemm_bi(a, w, c)
    cf = torch.empty((512, N), dtype=torch.float32, device=DEV)
    biv.gemm_bi(a, w, cf)
    sync()
    ref = oracle.linear(oracle.as_f64(a_np, "bf16"), oracle.as_f64(w_np, "bf16"))
    check_bf16(f64(c), ref, "gemm bf16 out")
    check_f32(f64(cf), ref, axis=1, what="gemm fp32 out")
    full = bits(c)
    for M in M_SWEEP:
        cM = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
        biv.gemm_bi(a[:M].contiguous(), w, cM)
        sync()
        assert np.array_equal(bits(cM), full[:M]), f"rows changed at M={M}"
    perm = wl.rng(2).permutation(512)
    cp = torch.empty_like(c)
    biv.gemm_bi(a[torch.from_numpy(perm).to(DEV)].contiguous(), w, cp)
    sync()
    assert np.array_equal(bits(cp), full[perm])


def _swiglu_ref(a_np, wg_np, wu_np):
    a = oracle.as_f64(a_np, "bf16")
    return oracle.silu(oracle.linear(a, oracle.as_f64(wg_np, "bf16"))) * oracle.linear(a, oracle.as_f64(wu_np, "bf16"))


def test_gemm_swiglu_epilogue_parity_and_invariance(biv):
    """gate/up in one product with SwiGLU applied to the fp32 results:
    silu(A Wg^T) * (A Wu^T) against the fp64 oracle (bf16 and fp32 outputs),
    and every row's bits identical for M = 1 .. 512."""
    M, F, K = 512, 2048, 4096
    a_np = wl.normal_bf16(60, (M, K))
    wg_np = wl.normal_bf16(61, (F, K), std=0.02)
    wu_np = wl.normal_bf16(62, (F, K), std=0.02)
    a = dev_bf16(a_np)
    w = biv.pack_gate_up(dev_bf16(np.concatenate([wg_np, wu_np], axis=0)))
    announce("gemm swiglu epilogue", M, F, K)
    c = torch.empty((M, F), dtype=torch.bfloat16, device=DEV)
    biv.gemm_bi(a, w, c, swiglu=True)
    cf = torch.empty((M, F), dtype=torch.float32, device=DEV)
    biv.gemm_bi(a, w, cf, swiglu=True)
    sync()
    ref = _swiglu_ref(a_np, wg_np, wu_np)
    check_bf16(f64(c), ref, "swiglu epilogue bf16")
    check_f32(f64(cf), ref, axis=1, what="swiglu epilogue fp32")
    full = bits(c)
    for m in M_SWEEP:
        cm = torch.empty((m, F), dtype=torch.bfloat16, device=DEV)
        biv.gemm_bi(a[:m].contiguous(), w, cm, swiglu=True)
        sync()
        assert np.array_equal(bits(cm), full[:m]), f"rows changed at M={m}"


def test_gemm_swiglu_epilogue_ragged_and_unfused_layout(biv):
    """A ragged shape (M and F not multiples of the tile) against the oracle,
    and the unfused route over the same packed weight (GEMM, then swiglu with
    block 32) within the same tolerance."""
    M, F, K = 77, 96, 320
    a_np = wl.normal_bf16(63, (M, K))
    wg_np = wl.normal_bf16(64, (F, K), std=0.05)
    wu_np = wl.normal_bf16(65, (F, K), std=0.05)
    a = dev_bf16(a_np)
    w = biv.pack_gate_up(dev_bf16(np.concatenate([wg_np, wu_np], axis=0)))
    announce("gemm swiglu ragged", M, F, K)
    c = torch.empty((M, F), dtype=torch.float32, device=DEV)
    biv.gemm_bi(a, w, c, swiglu=True)
    gu = torch.empty((M, 2 * F), dtype=torch.float32, device=DEV)
    biv.gemm_bi(a, w, gu)
    c2 = torch.empty((M, F), dtype=torch.float32, device=DEV)
    biv.swiglu(gu, c2, block=biv.SWIGLU_BLOCK)
    sync()
    ref = _swiglu_ref(a_np, wg_np, wu_np)
    check_f32(f64(c), ref, axis=1, what="swiglu ragged")
    check_f32(f64(c2), ref, axis=1, what="swiglu unfused over the packed weight")


@pytest.mark.parametrize("N", [4096, 6144, 6184, 14336, 28672])
def test_gemm_bf16_tile_classes_invariance(biv, N):
    """Each weight-width class of the staged kernel (its own column tiling:
    N <= 4096, 4096 < N < 8192 with 6184 ragged against the tile,
    8192 <= N < 16384, N >= 16384), K = 4096: parity with the oracle at
    M = 333 (ragged rows), and every row's bits the same for M = 1, 7, 32, 33,
    64, 65, 333 as inside M = 512 -- across the 32-row (M <= 32), 64-row
    (M <= 64) and full-height tiles."""
    K = 4096
    a_np = wl.normal_bf16(130, (512, K))
    w_np = wl.normal_bf16(131 + N % 7, (N, K), std=0.02)
    a, w = dev_bf16(a_np), dev_bf16(w_np)
    announce("gemm bf16 tile class", N)
    full = torch.empty((512, N), dtype=torch.float32, device=DEV)
    biv.gemm_bi(a, w, full)
    sync()
    full_bits = bits(full)
    ref = oracle.linear(oracle.as_f64(a_np[:333], "bf16"), oracle.as_f64(w_np, "bf16"))
    check_f32(f64(full)[:333], ref, axis=1, what=f"gemm N={N}")
    for M in (1, 7, 32, 33, 64, 65, 333):
        cM = torch.empty((M, N), dtype=torch.float32, device=DEV)
        biv.gemm_bi(a[:M].contiguous(), w, cM)
        sync()
        assert np.array_equal(bits(cM), full_bits[:M]), f"rows changed at M={M}, N={N}"


def test_gemm_bf16_down_projection_shape(biv):
    """The pass's longest reduction: the down projection [M, 14336] x
    [4096, 14336]^T (224 k-stages of 64) with the residual-accumulate
    epilogue into an fp32 stream, as the decoder calls it.  Parity with the
    oracle (fp32 output, per-row relative bound) at M = 512, and every row's
    bits the same at M = 1, 7, 32, 33, 64, 65 (the 32- and 64-row tiles) as
    inside M = 512 (the 128-row tile)."""
    M, N, K = 512, 4096, 14336
    a_np = wl.normal_bf16(190, (M, K), std=1.0)
    w_np = wl.normal_bf16(191, (N, K), std=0.02)
    r_np = wl.normal_f32(192, (M, N), std=3.0)
    a, w = dev_bf16(a_np), dev_bf16(w_np)
    announce("gemm bf16 down projection shape", M, N, K)
    full = dev_f32(r_np)
    biv.gemm_bi(a, w, full, accumulate=True)
    sync()
    ref = r_np.astype(np.float64) + oracle.linear(oracle.as_f64(a_np, "bf16"), oracle.as_f64(w_np, "bf16"))
    check_f32(f64(full), ref, axis=1, what="down projection + residual")
    full_bits = bits(full)
    for m in (1, 7, 32, 33, 64, 65):
        cm = dev_f32(r_np[:m])
        biv.gemm_bi(a[:m].contiguous(), w, cm, accumulate=True)
        sync()
        assert np.array_equal(bits(cm), full_bits[:m]), f"rows changed at M={m}"
    # bf16 output of the same product (store epilogue): R16 bf16 bound
    cb = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    biv.gemm_bi(a, w, cb)
    sync()
    check_bf16(f64(cb), ref - r_np.astype(np.float64), "down projection bf16 out")


@pytest.mark.parametrize("K", [4096, 4160])
def test_gemm_bf16_tiles_and_k_widths_change_no_bits(biv, K):
    """One weight of 6144 rows (the 128 x 96 tile class: 128-wide k stages
    when K % 128 == 0, else 64-wide) against its column slices of 4096 and
    2048 rows (the 128 x 64 tile, 64-wide k stages): every output element is
    reduced in the same order whatever tile and k width hold it, so the
    columns agree bit for bit (fp32 and bf16 outputs); the same rows at
    M = 5 and 40 (32- and 64-row tiles) match too."""
    M, N = 333, 6144
    a_np = wl.normal_bf16(140, (M, K))
    w_np = wl.normal_bf16(141, (N, K), std=0.02)
    a, w = dev_bf16(a_np), dev_bf16(w_np)
    announce("gemm tiles and k widths", K)
    for dt in (torch.float32, torch.bfloat16):
        full = torch.empty((M, N), dtype=dt, device=DEV)
        biv.gemm_bi(a, w, full)
        lo = torch.empty((M, 4096), dtype=dt, device=DEV)
        hi = torch.empty((M, N - 4096), dtype=dt, device=DEV)
        biv.gemm_bi(a, w[:4096].contiguous(), lo)
        biv.gemm_bi(a, w[4096:].contiguous(), hi)
        sync()
        fb = bits(full)
        assert np.array_equal(bits(lo), fb[:, :4096]), f"K={K} {dt}: columns 0..4095"
        assert np.array_equal(bits(hi), fb[:, 4096:]), f"K={K} {dt}: columns 4096.."
        for m in (5, 40):  # the 32- and 64-row tiles of both classes, both k widths
            part = torch.empty((m, N), dtype=dt, device=DEV)
            biv.gemm_bi(a[:m].contiguous(), w, part)
            sync()
            assert np.array_equal(bits(part), fb[:m]), f"K={K} {dt}: rows changed at M={m}"
    ref = oracle.linear(oracle.as_f64(a_np, "bf16"), oracle.as_f64(w_np, "bf16"))
    check_bf16(f64(full), ref, f"gemm tiles K={K}")


@pytest.mark.parametrize("M,N,K", [(77, 200, 264), (1, 130, 8), (129, 257, 1000), (300, 128, 4096)])
def test_gemm_bf16_ragged_shapes(biv, M, N, K):
    a_np = wl.normal_bf16(20 + M, (M, K))
    w_np = wl.normal_bf16(21 + N, (N, K), std=0.05)
    c = torch.empty((M, N), dtype=torch.float32, device=DEV)
    announce("gemm bf16 ragged", M, N, K)
    biv.gemm_bi(dev_bf16(a_np), dev_bf16(w_np), c)
    sync()
    ref = oracle.linear(oracle.as_f64(a_np, "bf16"), oracle.as_f64(w_np, "bf16"))
    check_f32(f64(c), ref, axis=1, what="ragged gemm")


@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_gemm_accumulate_epilogue(biv, out):
    M, N, K = 64, 256, 512
    a_np = wl.normal_bf16(30, (M, K))
    w_np = wl.normal_bf16(31, (N, K), std=0.05)
    r_np = wl.normal_f32(32, (M, N))
    if out == "f32":
        c = dev_f32(r_np)
        r64 = r_np.astype(np.float64)
    else:
        rb = wl.bf16_bits(r_np)
        c = dev_bf16(rb)
        r64 = oracle.as_f64(rb, "bf16")
    announce("gemm accumulate", out)
    biv.gemm_bi(dev_bf16(a_np), dev_bf16(w_np), c, accumulate=True)
    sync()
    ref = r64 + oracle.linear(oracle.as_f64(a_np, "bf16"), oracle.as_f64(w_np, "bf16"))
    if out == "f32":
        check_f32(f64(c), ref, axis=1, what="accumulate f32")
    else:
        check_bf16(f64(c), ref, "accumulate bf16")


def test_gemm_f32_parity_and_invariance(biv):
    M, N, K = 16, 1024, 256
    a_np = wl.normal_f32(40, (M, K))
    w_np = wl.normal_f32(41, (N, K), std=0.02)
    a, w = dev_f32(a_np), dev_f32(w_np)
    c = torch.empty((M, N), dtype=torch.float32, device=DEV)
    announce("gemm f32")
    biv.gemm_bi(a, w, c)
    sync()
    check_f32(f64(c), oracle.linear(a_np, w_np), axis=1, what="gemm f32")
    full = bits(c)
    for m in range(1, M + 1):
        cm = torch.empty((m, N), dtype=torch.float32, device=DEV)
        biv.gemm_bi(a[:m].contiguous(), w, cm)
        sync()
        assert np.array_equal(bits(cm), full[:m])
    # ragged K and N on the fp32 path
    a2 = wl.normal_f32(42, (5, 37))
    w2 = wl.normal_f32(43, (70, 37))
    c2 = torch.empty((5, 70), dtype=torch.float32, device=DEV)
    biv.gemm_bi(dev_f32(a2), dev_f32(w2), c2)
    sync()
    check_f32(f64(c2), oracle.linear(a2, w2), axis=1, what="gemm f32 ragged")


# =====================================================================
# attn_decode_bi
# =====================================================================


def _attn_inputs(R, q_len, Hq, Hkv, D, ctx, seed, dtype="bf16", spare=3):
    lay = wl.paged_layout(ctx, q_len, seed=seed, spare_blocks=spare)
    mk = wl.normal_bf16 if dtype == "bf16" else wl.normal_f32
    kc = mk(seed + 1, (lay.num_blocks, Hkv, 16, D))
    vc = mk(seed + 2, (lay.num_blocks, Hkv, 16, D))
    q = mk(seed + 3, (R * q_len, Hq, D))
    return lay, kc, vc, q


def _run_attn(biv, lay, kc, vc, q, q_len, dtype="bf16", fn=None, **kw):
    dev = dev_bf16 if dtype == "bf16" else dev_f32
    T, Hq, D = q.shape
    out = torch.full((T, Hq, D), float("nan"), dtype=torch.bfloat16 if dtype == "bf16" else torch.float32,
                     device=DEV)
    kcd, vcd = dev(kc), dev(vc)
    bt, cx = dev_i32(lay.block_table), dev_i32(lay.ctx)
    ws = None
    if dtype == "bf16":
        seg = kw.pop("seg", None)
        nbytes = biv.attn_workspace_bytes(len(lay.ctx), kc.shape[1], lay.max_blocks,
                                          seg if seg is not None else biv.ATTN_SEG_TOKENS, q_len=q_len, Hq=Hq)
        ws = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    (fn or biv.attn_decode_bi)(dev(q), kcd, vcd, bt, cx, out, q_len, 1.0 / math.sqrt(D), ws, **kw)
    sync()
    return out


def _attn_ref(lay, kc, vc, q, q_len, dtype="bf16"):
    return oracle.attention(oracle.as_f64(q, dtype), oracle.as_f64(kc, dtype), oracle.as_f64(vc, dtype),
                            lay.block_table, lay.ctx, q_len, 1.0 / math.sqrt(q.shape[-1]))


@pytest.mark.parametrize("q_len", [1, 8])
def test_attention_bf16_parity(biv, q_len):
    """32 q heads / 8 KV heads x 128, paged KV (16-token pages, permuted),
    contexts spanning several 256-token chunks and 4096-token segments plus
    ragged tails and exact boundaries (sub-tile, chunk and segment ends; 15
    requests: segments split over several waves)."""
    ctx = [0, 255 - q_len + 1, 256, 512 - q_len, 513 - q_len, 1023, 1024, 1025, 2048 - q_len, 2049 - q_len, 2500,
           4096 - q_len, 4097 - q_len, 5000, 9000]
    R = len(ctx)
    lay, kc, vc, q = _attn_inputs(R, q_len, 32, 8, 128, ctx, seed=50 + q_len)
    announce("attention bf16 parity q_len", q_len)
    out = _run_attn(biv, lay, kc, vc, q, q_len)
    ref = _attn_ref(lay, kc, vc, q, q_len)
    check_bf16(f64(out), ref, f"attention bf16 q_len={q_len}")
    # a single visible key returns its value exactly
    v0 = oracle.as_f64(vc, "bf16")[lay.block_table[0, 0], :, 0, :]  # [Hkv, D]
    got = f64(out)[0]  # request 0, row 0
    for h in range(32):
        assert np.array_equal(got[h], v0[h // 4])


def test_attention_bf16_batch_invariance(biv):
    """Request 0's outputs are bit-identical alone, at another batch slot,
    with other requests next to it, and with its pages elsewhere in memory."""
    q_len, Hq, Hkv, D = 8, 32, 8, 128
    base_ctx = 3000
    lay, kc, vc, q = _attn_inputs(1, q_len, Hq, Hkv, D, [base_ctx], seed=60)
    announce("attention invariance alone")
    alone = bits(_run_attn(biv, lay, kc, vc, q, q_len))
    g = wl.rng(61)
    for trial in range(3):
        R = int(g.integers(2, 12))
        slot = int(g.integers(0, R))
        ctx = list(g.integers(500, 9000, size=R))
        ctx[slot] = base_ctx
        lay2 = wl.paged_layout(ctx, q_len, seed=62 + trial, spare_blocks=int(g.integers(0, 9)))
        kc2 = wl.normal_bf16(63 + trial, (lay2.num_blocks, Hkv, 16, D))
        vc2 = wl.normal_bf16(64 + trial, (lay2.num_blocks, Hkv, 16, D))
        q2 = wl.normal_bf16(65 + trial, (R * q_len, Hq, D))
        # copy request 0's pages and queries into the new layout at `slot`
        for b in range(lay.max_blocks):
            src, dst = lay.block_table[0, b], lay2.block_table[slot, b]
            if src >= 0:
                kc2[dst] = kc[src]
                vc2[dst] = vc[src]
        q2[slot * q_len:(slot + 1) * q_len] = q
        announce("attention invariance trial", trial, R, slot)
        out2 = bits(_run_attn(biv, lay2, kc2, vc2, q2, q_len))
        assert np.array_equal(out2[slot * q_len:(slot + 1) * q_len], alone), f"trial {trial}"



@pytest.mark.parametrize("q_len", [1, 8])
def test_attention_split_segments_equal_unsplit(biv, q_len):
    """A request alone is few segment waves, so each segment is split over
    16 waves (later parts store per-chunk partials, completed by the chunk
    fold before the segment fold); beside 63 other requests the grid holds
    at least 1024 waves and nothing is split.  Its rows are the same bits
    either way, across a split single segment, a part left without keys, a
    ragged last chunk and exact segment boundaries."""
    Hq, Hkv, D = 32, 8, 128
    for L in (300, 4096 - q_len, 4097 - q_len, 5000, 9000, 12290):
        lay, kc, vc, q = _attn_inputs(1, q_len, Hq, Hkv, D, [L], seed=95)
        announce("attention split vs unsplit, alone", q_len, L)
        alone = bits(_run_attn(biv, lay, kc, vc, q, q_len))
        slot, R = 7, 64
        ctx = [100] * R
        ctx[slot], ctx[11] = L, 4200  # one filler past 4096 keys: at least two segments per request
        lay2 = wl.paged_layout(ctx, q_len, seed=96, spare_blocks=2)
        assert R * Hkv * -(-lay2.max_blocks * 16 // biv.ATTN_SEG_TOKENS) >= 1024  # unsplit grid
        kc2 = wl.normal_bf16(97, (lay2.num_blocks, Hkv, 16, D))
        vc2 = wl.normal_bf16(98, (lay2.num_blocks, Hkv, 16, D))
        q2 = wl.normal_bf16(99, (R * q_len, Hq, D))
        for b in range(lay.max_blocks):
            src, dst = lay.block_table[0, b], lay2.block_table[slot, b]
            if src >= 0:
                kc2[dst] = kc[src]
                vc2[dst] = vc[src]
        q2[slot * q_len:(slot + 1) * q_len] = q
        announce("attention split vs unsplit, batched", q_len, L)
        out2 = bits(_run_attn(biv, lay2, kc2, vc2, q2, q_len))
        assert np.array_equal(out2[slot * q_len:(slot + 1) * q_len], alone), (q_len, L)

@pytest.mark.parametrize("q_len", [1, 8])
def test_attention_rows_equal_across_split_counts(biv, q_len):
    """The same request in batches of 1, 8, 16, 32 and 64 over one block
    table (three 4096-token segments per request at most) is taken by 16, 8,
    4, 2 and 1 waves per segment: parts of one 256-token chunk, of several
    chunks, and no split.  Its rows are the same bits in every batch."""
    Hq, Hkv, D, R = 32, 8, 128, 64
    ctx = [9000] + list(wl.rng(310).integers(50, 3000, size=R - 1))
    lay, kc, vc, q = _attn_inputs(R, q_len, Hq, Hkv, D, ctx, seed=311)
    nseg_max = -(-lay.max_blocks * 16 // biv.ATTN_SEG_TOKENS)
    assert nseg_max == 3
    kcd, vcd, qd = dev_bf16(kc), dev_bf16(vc), dev_bf16(q)
    bt_all, cx_all = dev_i32(lay.block_table), dev_i32(lay.ctx)
    rows = {}
    for B in (1, 8, 16, 32, 64):
        potential, parts = B * Hkv * nseg_max, 1
        while 16 % (2 * parts) == 0 and potential * parts < 1024:
            parts *= 2
        announce("attention split counts", q_len, B, parts)
        out = torch.full((B * q_len, Hq, D), float("nan"), dtype=torch.bfloat16, device=DEV)
        ws = torch.zeros(biv.attn_workspace_bytes(B, Hkv, lay.max_blocks, q_len=q_len, Hq=Hq), dtype=torch.uint8,
                         device=DEV)
        biv.attn_decode_bi(qd[:B * q_len], kcd, vcd, bt_all[:B].contiguous(), cx_all[:B].contiguous(), out, q_len,
                           1.0 / math.sqrt(D), ws)
        sync()
        rows[parts] = bits(out)[:q_len].copy()
    assert sorted(rows) == [1, 2, 4, 8, 16]
    for parts, r in rows.items():
        assert np.array_equal(r, rows[1]), (q_len, parts)


def test_attention_bf16_verify_rows_equal_single_decodes(biv):
    """Row j of a K=8 verify block equals, bit for bit, the same query decoded
    alone (K=1) at context L+j: extra masked keys and chunks fold as no-ops."""
    q_len, Hq, Hkv, D, L = 8, 32, 8, 128, 4090  # crosses a chunk and a segment boundary
    lay, kc, vc, q = _attn_inputs(1, q_len, Hq, Hkv, D, [L], seed=70)
    announce("attention verify vs decode")
    block = bits(_run_attn(biv, lay, kc, vc, q, q_len))
    for j in range(q_len):
        lay1 = wl.PagedLayout(ctx=np.array([L + j], np.int32), q_len=1, block_table=lay.block_table,
                              num_blocks=lay.num_blocks, max_blocks=lay.max_blocks)
        one = bits(_run_attn(biv, lay1, kc, vc, q[j:j + 1], 1))
        assert np.array_equal(one[0], block[j]), f"row {j}"


@pytest.mark.parametrize("G", [2, 8, 32])
@pytest.mark.parametrize("q_len", [1, 8])
def test_attention_bf16_gqa_ratios(biv, q_len, G):
    """Other query-to-KV head ratios G (dividing 32): a 32-row block then holds
    32/G positions of G heads (16, 4 or 1 positions), so a verify step of 8
    positions takes 1, 2 or 8 row blocks.  Parity with the oracle on contexts
    from empty to three segments, and each request alone (its segments split
    over more waves) the same bits as in the batch."""
    Hkv = 2
    Hq = Hkv * G
    ctx = [0, 300, 4097 - q_len, 9000]
    lay, kc, vc, q = _attn_inputs(len(ctx), q_len, Hq, Hkv, 128, ctx, seed=400 + G + q_len)
    announce("attention bf16 GQA ratio", G, q_len)
    out = _run_attn(biv, lay, kc, vc, q, q_len)
    check_bf16(f64(out), _attn_ref(lay, kc, vc, q, q_len), f"attention bf16 G={G} q_len={q_len}")
    full = bits(out)
    for r in (1, 3):
        lay1 = wl.PagedLayout(ctx=lay.ctx[r:r + 1], q_len=q_len, block_table=lay.block_table[r:r + 1],
                              num_blocks=lay.num_blocks, max_blocks=lay.max_blocks)
        one = bits(_run_attn(biv, lay1, kc, vc, q[r * q_len:(r + 1) * q_len], q_len))
        assert np.array_equal(one, full[r * q_len:(r + 1) * q_len]), f"G={G} q_len={q_len} request {r}"


@pytest.mark.parametrize("q_len,G", [(33, 4), (200, 4), (70, 1)])
def test_attention_bf16_row_blocks_prefill(biv, q_len, G):
    """q_len beyond one 32-row block (a prefill, or a long verify): the rows
    are taken 32/G positions at a time, each block with the keys up to its own
    last row.  Parity with the oracle (contexts 0 -- a causal prefill -- and
    across chunk and segment boundaries), and sampled rows bit for bit those of
    single-row decodes at context L + j."""
    Hkv = 8 if G == 4 else 4
    Hq = Hkv * G
    ctx = [0, 700, 2300]
    R = len(ctx)
    lay, kc, vc, q = _attn_inputs(R, q_len, Hq, Hkv, 128, ctx, seed=150 + q_len + G)
    announce("attention bf16 row blocks", q_len, G)
    out = _run_attn(biv, lay, kc, vc, q, q_len)
    check_bf16(f64(out), _attn_ref(lay, kc, vc, q, q_len), f"attention bf16 q_len={q_len} G={G}")
    full = bits(out)
    blk = 32 // G
    for r in range(R):
        for j in sorted({0, blk - 1, blk, q_len // 2, q_len - 1}):
            lay1 = wl.PagedLayout(ctx=np.array([ctx[r] + j], np.int32), q_len=1, block_table=lay.block_table[r:r + 1],
                                  num_blocks=lay.num_blocks, max_blocks=lay.max_blocks)
            one = bits(_run_attn(biv, lay1, kc, vc, q[r * q_len + j:r * q_len + j + 1], 1))
            assert np.array_equal(one[0], full[r * q_len + j]), f"request {r} row {j}"


def _ragged_case(biv, ctx, qlens, Hq, Hkv, D, seed, dtype="bf16"):
    """Requests with their own row counts (q_off), laid out back to back; returns
    (layout, caches, q, offsets, output bits, output values)."""
    qmax = max(qlens)
    lay = wl.paged_layout(ctx, qmax, seed=seed, spare_blocks=2)
    mk = wl.normal_bf16 if dtype == "bf16" else wl.normal_f32
    kc = mk(seed + 1, (lay.num_blocks, Hkv, 16, D))
    vc = mk(seed + 2, (lay.num_blocks, Hkv, 16, D))
    off = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    q = mk(seed + 3, (int(off[-1]), Hq, D))
    out = _run_attn(biv, lay, kc, vc, q, qmax, dtype=dtype, q_off=dev_i32(off))
    return lay, kc, vc, q, off, bits(out), f64(out)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_attention_ragged_rows_q_off(biv, dtype):
    """attn_decode_bi with per-request row offsets (requests bring different
    numbers of candidates, one none): every request's rows match the oracle and
    equal, bit for bit, that request run alone with a uniform q_len; a
    request's rows do not change when its neighbours' row counts change."""
    Hq, Hkv, D = (32, 8, 128) if dtype == "bf16" else (4, 4, 64)
    ctx = [700, 4090, 0, 2500, 9000, 300]
    qlens = [1, 8, 5, 20, 0, 3]  # 20 rows at G = 4: three 8-position row blocks
    announce("attention ragged rows", dtype, qlens)
    lay, kc, vc, q, off, ob, ov = _ragged_case(biv, ctx, qlens, Hq, Hkv, D, seed=170, dtype=dtype)
    chk = (lambda g, r, w: check_bf16(g, r, w)) if dtype == "bf16" else (lambda g, r, w: check_f32(g, r, what=w))
    for r, n in enumerate(qlens):
        if n == 0:
            continue
        rows = q[off[r]:off[r + 1]]
        lay1 = wl.PagedLayout(ctx=np.array([ctx[r]], np.int32), q_len=n, block_table=lay.block_table[r:r + 1],
                              num_blocks=lay.num_blocks, max_blocks=lay.max_blocks)
        chk(ov[off[r]:off[r + 1]], _attn_ref(lay1, kc, vc, rows, n, dtype), f"ragged request {r}")
        alone = bits(_run_attn(biv, lay1, kc, vc, rows, n, dtype=dtype))
        assert np.array_equal(ob[off[r]:off[r + 1]], alone), f"request {r} differs from running alone"
    # the neighbours' row counts change (same caches and pages); request 3
    # (20 rows) keeps its bits
    qlens2 = [8, 2, 1, 20, 7, 8]
    off2 = np.concatenate([[0], np.cumsum(qlens2)]).astype(np.int32)
    mk = wl.normal_bf16 if dtype == "bf16" else wl.normal_f32
    q2 = mk(180, (int(off2[-1]), Hq, D))
    q2[off2[3]:off2[4]] = q[off[3]:off[4]]
    announce("attention ragged rows, other neighbours", dtype, qlens2)
    out2 = _run_attn(biv, lay, kc, vc, q2, max(qlens2), dtype=dtype, q_off=dev_i32(off2))
    assert np.array_equal(bits(out2)[off2[3]:off2[4]], ob[off[3]:off[4]])


def test_attention_f32_parity(biv):
    """fp32 path (tiny model: 4 heads x 64, no grouping), decode, verify and
    prefill-shaped calls."""
    for q_len, ctx in [(1, [0, 5, 300]), (4, [128, 17, 600]), (128, [0])]:
        R = len(ctx)
        lay, kc, vc, q = _attn_inputs(R, q_len, 4, 4, 64, ctx, seed=80 + q_len, dtype="f32")
        announce("attention f32", q_len, ctx)
        out = _run_attn(biv, lay, kc, vc, q, q_len, dtype="f32")
        check_f32(f64(out), _attn_ref(lay, kc, vc, q, q_len, "f32"), what=f"attention f32 q_len={q_len}")


def test_attention_adaptive_matches_oracle(biv):
    q_len = 1
    ctx = [600, 4000, 9000, 12000]
    lay, kc, vc, q = _attn_inputs(len(ctx), q_len, 32, 8, 128, ctx, seed=90)
    split = biv.attn_adaptive_split(len(ctx), 8, lay.max_blocks)
    announce("attention adaptive split", split)
    out = _run_attn(biv, lay, kc, vc, q, q_len, fn=biv.attn_decode_adaptive, seg=split)
    check_bf16(f64(out), _attn_ref(lay, kc, vc, q, q_len), "attention adaptive")



def test_attention_adaptive_any_split_fits_smallest_split_workspace(biv):
    """The load-adaptive call never splits a segment over waves, so a
    workspace sized for its smallest segment (256 tokens: the most segment
    partials) serves every larger one -- what a comparison pass that times
    several splits with one workspace relies on; each split still matches
    the oracle."""
    q_len = 8
    ctx = [600, 4000, 9000]  # few requests: the invariant call would split these segments
    lay, kc, vc, q = _attn_inputs(len(ctx), q_len, 32, 8, 128, ctx, seed=91)
    ws = torch.empty(biv.attn_workspace_bytes(len(ctx), 8, lay.max_blocks, 256), dtype=torch.uint8, device=DEV)
    ref = _attn_ref(lay, kc, vc, q, q_len)
    qd, kcd, vcd = dev_bf16(q), dev_bf16(kc), dev_bf16(vc)
    bt, cx = dev_i32(lay.block_table), dev_i32(lay.ctx)
    for split in (256, 512, 1024, 2048, 4096, 8192):
        announce("attention adaptive, one workspace, split", split)
        out = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device=DEV)
        biv.attn_decode_adaptive(qd, kcd, vcd, bt, cx, out, q_len, 1.0 / math.sqrt(128), ws, split_tokens=split)
        sync()
        check_bf16(f64(out), ref, f"attention adaptive split {split}")

# =====================================================================
# split-K, RoPE, SwiGLU, embedding
# =====================================================================


@pytest.mark.parametrize("M", [1, 16, 512])
def test_gemm_splitk_matches_oracle(biv, M):
    K, N = 4096, 2048
    a_np = wl.normal_bf16(100 + M, (M, K))
    w_np = wl.normal_bf16(101, (N, K), std=0.02)
    sp = biv.splitk_auto_splits(M, N, K)
    ws = torch.empty(biv.splitk_workspace_bytes(M, N, sp) // 4 + 1, dtype=torch.float32, device=DEV)
    c = torch.empty((M, N), dtype=torch.float32, device=DEV)
    announce("gemm splitk", M, sp)
    biv.gemm_splitk(dev_bf16(a_np), dev_bf16(w_np), c, 0, ws)
    sync()
    ref = oracle.linear(oracle.as_f64(a_np, "bf16"), oracle.as_f64(w_np, "bf16"))
    check_f32(f64(c), ref, axis=1, what="splitk")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rope_swiglu_embed(biv, dtype):
    dev = dev_bf16 if dtype == "bf16" else dev_f32
    mk = wl.normal_bf16 if dtype == "bf16" else wl.normal_f32
    chk = (lambda g, r, w: check_bf16(g, r, w)) if dtype == "bf16" else (lambda g, r, w: check_f32(g, r, what=w))
    T, H, D = 9, 6, 128
    x_np = mk(110, (T, (H + 2) * D))
    pos = np.array([0, 1, 7, 100, 2047, 5000, 8191, 30000, 65535], np.int32)
    x = dev(x_np)
    table = biv.rope_table(65536, D, 500000.0).to(DEV)
    announce("rope", dtype)
    biv.rope_apply(x, dev_i32(pos), table, H, D)
    sync()
    ref = oracle.as_f64(x_np, dtype).copy()
    ref[:, :H * D] = oracle.rope(ref[:, :H * D].reshape(T, H, D), pos, 500000.0).reshape(T, H * D)
    chk(f64(x), ref, "rope")
    gu_np = mk(111, (33, 2 * 300))
    out = torch.empty((33, 300), dtype=x.dtype, device=DEV)
    biv.swiglu(dev(gu_np), out)
    sync()
    gu = oracle.as_f64(gu_np, dtype)
    chk(f64(out), oracle.silu(gu[:, :300]) * gu[:, 300:], "swiglu")
    # interleaved layout: groups of 2*30 columns, gate 30 then up 30
    outb = torch.empty((33, 300), dtype=x.dtype, device=DEV)
    biv.swiglu(dev(gu_np), outb, block=30)
    sync()
    n = np.arange(300)
    gi = 60 * (n // 30) + n % 30
    chk(f64(outb), oracle.silu(gu[:, gi]) * gu[:, gi + 30], "swiglu block 30")
    tab_np = mk(112, (50, 64))
    ids = np.array([3, 49, 0, 7, -1, 50], np.int32)
    emb = torch.empty((6, 64), dtype=torch.float32, device=DEV)
    biv.embed_rows(dev_i32(ids), dev(tab_np), emb)
    sync()
    ref = np.zeros((6, 64))
    ref[:4] = oracle.as_f64(tab_np, dtype)[ids[:4]]
    assert np.array_equal(f64(emb), ref)
    # output in the table's dtype, and a width that is not a multiple of 8
    # (bf16: the 16-byte path above, the element loop here)
    emb_t = torch.empty((6, 64), dtype=x.dtype, device=DEV)
    biv.embed_rows(dev_i32(ids), dev(tab_np), emb_t)
    tab2_np = mk(113, (50, 60))
    emb2 = torch.empty((6, 60), dtype=torch.float32, device=DEV)
    biv.embed_rows(dev_i32(ids), dev(tab2_np), emb2)
    sync()
    assert np.array_equal(f64(emb_t), ref)
    ref2 = np.zeros((6, 60))
    ref2[:4] = oracle.as_f64(tab2_np, dtype)[ids[:4]]
    assert np.array_equal(f64(emb2), ref2)
