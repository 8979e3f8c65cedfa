"""Pins of the CPU oracle to facts fixed by the pages and by mathematics.

Each test checks the oracle against something other than itself: hand-built
vectors from the pages, closed forms, brute-force searches, exact rational
arithmetic, invariants and independent library routines.  A plausible mistake
in the oracle (a dropped term, a wrong sign or index, a transposed operand, a
wrong Qmax, a symmetric instead of asymmetric range, a swapped nibble order)
fails at least one of them.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import synth_inputs as SI
from oracle import lbq_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
F32 = np.float32


def _f32_ulp(x):
    x = np.abs(np.asarray(x, dtype=F32))
    return (np.nextafter(x, F32(np.inf)) - x).astype(np.float64)


# ---------------------------------------------------------------- packing

def _packing_rows():
    rows = []
    with open(os.path.join(GOLDEN, "packing_vectors.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            b, codes, packed = [p.strip() for p in line.split("|")]
            rows.append((int(b), [int(c) for c in codes.split()],
                         [int(h, 16) for h in packed.split()]))
    return rows


@pytest.mark.parametrize("bits,codes,expect", _packing_rows())
def test_packing_golden_vectors(bits, codes, expect):
    got = O.pack_codes(np.array([codes], dtype=np.uint8), bits)[0]
    assert list(got) == expect
    back = O.unpack_codes(np.array([expect], dtype=np.uint8), bits)[0]
    assert list(back) == codes


@pytest.mark.parametrize("bits", [2, 4])
def test_unpack_pack_identity(bits):
    rng = np.random.default_rng(7)
    codes = rng.integers(0, 1 << bits, size=(5, 64)).astype(np.uint8)
    assert np.array_equal(O.unpack_codes(O.pack_codes(codes, bits), bits), codes)
    raw = rng.integers(0, 256, size=(3, 16)).astype(np.uint8)
    assert np.array_equal(O.pack_codes(O.unpack_codes(raw, bits), bits), raw)


# ---------------------------------------------------------------- bf16

def test_bf16_matches_torch_cpu_conversion():
    import torch
    rng = np.random.default_rng(11)
    x = np.concatenate([
        rng.standard_normal(1_000_000).astype(F32) * F32(3.0),
        (rng.standard_normal(20000) * 1e-38).astype(F32),       # subnormals
        (rng.standard_normal(20000) * 1e30).astype(F32),
        np.array([0.0, -0.0, 1.0, -1.0, 3.4e38, -3.4e38, 1e-45], dtype=F32),
    ])
    # exact ties: low 16 bits == 0x8000, both parities of the kept bit
    ties = (rng.integers(0x0080, 0x7F00, size=4000, dtype=np.uint32) << np.uint32(16)) | np.uint32(0x8000)
    x = np.concatenate([x, ties.view(F32), (-ties.view(F32)).astype(F32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.bf16_bits(x), ref)
    assert np.array_equal(O.bf16_to_f64(ref), torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).double().numpy())


# ---------------------------------------------------------------- MinMax

CASES = [(4, 128), (2, 64), (4, 64), (2, 128)]


@pytest.mark.parametrize("bits,group", CASES)
def test_minmax_codes_are_nearest_level_bruteforce(bits, group):
    """With the stored (s, z), every code is the level (q - z)*s nearest to w
    among q in [0, Qmax], found by exhaustive fp64 search (ties excused)."""
    qmax = (1 << bits) - 1
    W = SI.gaussian_weights(101, 48, 4 * group, outlier_seed=102)
    codes, s, z = O.minmax_quantize(W, bits, group)
    N, K = W.shape
    w = W.astype(np.float64).reshape(N, K // group, group)
    levels = (np.arange(qmax + 1)[None, None, :] - z.astype(np.float64)[:, :, None]) * s.astype(np.float64)[:, :, None]
    dist = np.abs(w[..., None] - levels[:, :, None, :])
    best = dist.argmin(axis=-1)
    got = codes.reshape(best.shape).astype(np.int64)
    srt = np.sort(dist, axis=-1)
    near_tie = (srt[..., 1] - srt[..., 0]) <= 4 * _f32_ulp(w) + 1e-300
    bad = (best != got) & ~near_tie
    assert not bad.any()


@pytest.mark.parametrize("bits,group", CASES)
def test_minmax_scale_and_zero_closed_form(bits, group):
    """s*Qmax spans the group's range including 0 (to one fp32 rounding), the
    group minimum gets code 0 when it is negative and the maximum gets Qmax."""
    qmax = (1 << bits) - 1
    W = SI.gaussian_weights(103, 32, 4 * group, outlier_seed=104)
    codes, s, z = O.minmax_quantize(W, bits, group)
    N, K = W.shape
    Wg = W.astype(np.float64).reshape(N, K // group, group)
    cg = codes.reshape(N, K // group, group)
    span = np.maximum(0, Wg.max(-1)) - np.minimum(0, Wg.min(-1))
    assert np.all(np.abs(s.astype(np.float64) * qmax - span) <= span * 2.0 ** -22)
    # zero point: (0 - z) * s reproduces the group minimum to within s/2
    assert np.all(np.abs(-z.astype(np.float64) * s - np.minimum(0, Wg.min(-1))) <= 0.5 * s * (1 + 2.0 ** -20))
    imin = Wg.argmin(-1)[..., None]
    imax = Wg.argmax(-1)[..., None]
    assert np.all(np.take_along_axis(cg, imin, -1) == 0)
    assert np.all(np.take_along_axis(cg, imax, -1) == qmax)


@pytest.mark.parametrize("bits,group", CASES)
def test_minmax_error_bound(bits, group):
    """|w - (q - z) s| <= s (1/2 + 2^-18), in fp64 against the stored fp32 s."""
    W = np.concatenate([SI.gaussian_weights(105, 64, 512, outlier_seed=106),
                        SI.student_t_weights(107, 64, 512)])
    codes, s, z = O.minmax_quantize(W, bits, group)
    err = np.abs(W.astype(np.float64) - O.minmax_exact(codes, s, z, group))
    bound = np.repeat(s.astype(np.float64), group, axis=1) * (0.5 + 2.0 ** -18)
    assert np.all(err <= bound)


@pytest.mark.parametrize("bits,group", CASES)
def test_minmax_requantize_with_fixed_params_is_identity(bits, group):
    """quantize(dequantize(q)) == q with the stored (s, z) held fixed, both for
    the fp32 product and for the bf16-rounded dequantized weight."""
    W = SI.gaussian_weights(108, 40, 512, outlier_seed=109)
    codes, s, z = O.minmax_quantize(W, bits, group)
    N, K = W.shape
    qmax = (1 << bits) - 1
    srep = np.repeat(s, group, axis=1)
    zrep = np.repeat(z.astype(np.int32), group, axis=1)
    w32 = ((codes.astype(np.int32) - zrep).astype(F32) * srep).astype(F32)
    wbf = O.bf16_to_f64(O.minmax_dequant_bf16(codes, s, z, group)).astype(F32)
    for wh in (w32, wbf):
        q2 = np.clip(np.rint(wh / srep).astype(np.int32) + zrep, 0, qmax)
        assert np.array_equal(q2, codes.astype(np.int32))


def test_minmax_all_zero_weight():
    W = np.zeros((4, 256), dtype=F32)
    for bits, group in CASES:
        codes, s, z = O.minmax_quantize(W, bits, group)
        assert np.all(codes == 0) and np.all(z == 0) and np.all(s == 1)
        assert np.all(O.minmax_exact(codes, s, z, group) == 0)
        assert np.all(O.minmax_dequant_bf16(codes, s, z, group) == 0)


@pytest.mark.parametrize("bits,group", CASES)
def test_minmax_single_nonzero_per_group(bits, group):
    """One nonzero v per group: range [min(0,v), max(0,v)], so v > 0 gives
    z = 0, code(v) = Qmax, others 0; v < 0 gives z = Qmax, code(v) = 0, others Qmax."""
    qmax = (1 << bits) - 1
    rng = np.random.default_rng(110)
    N, K = 6, 4 * group
    W = np.zeros((N, K), dtype=F32)
    pos = rng.integers(0, group, size=(N, K // group))
    vals = (rng.uniform(0.01, 3.0, size=(N, K // group)) * np.where(rng.random((N, K // group)) < 0.5, -1, 1)).astype(F32)
    for i in range(N):
        for j in range(K // group):
            W[i, j * group + pos[i, j]] = vals[i, j]
    codes, s, z = O.minmax_quantize(W, bits, group)
    cg = codes.reshape(N, K // group, group)
    for i in range(N):
        for j in range(K // group):
            v = float(vals[i, j])
            assert s[i, j] == F32(abs(v)) / F32(qmax)
            if v > 0:
                assert z[i, j] == 0 and cg[i, j, pos[i, j]] == qmax
                assert np.count_nonzero(cg[i, j]) == 1
            else:
                assert z[i, j] == qmax and cg[i, j, pos[i, j]] == 0
                assert np.count_nonzero(cg[i, j] == qmax) == group - 1


@pytest.mark.parametrize("bits,group", CASES)
def test_minmax_power_of_two_grid_is_lossless(bits, group):
    W = SI.grid_weights(111, 8, 4 * group, group, bits, exp=4)
    codes, s, z = O.minmax_quantize(W, bits, group)
    assert np.all(s == F32(2.0 ** -4))
    assert np.array_equal(O.minmax_exact(codes, s, z, group), W.astype(np.float64))
    assert np.array_equal(O.bf16_to_f64(O.minmax_dequant_bf16(codes, s, z, group)), W.astype(np.float64))


def test_minmax_single_signed_group_range_includes_zero():
    """An all-positive group keeps lo = 0 (the reading that the range covers 0)."""
    W = np.full((1, 128), 0.5, dtype=F32)
    W[0, :64] = 0.2
    codes, s, z = O.minmax_quantize(W, 4, 128)
    assert z[0, 0] == 0 and s[0, 0] == F32(0.5) / F32(15)
    assert codes[0, 64] == 15 and codes[0, 0] == 6  # 0.2 / (0.5/15) = 6


# ---------------------------------------------------------------- NF4

def test_nf4_codebook_invariants():
    c = O.nf4_codebook()
    assert c.dtype == F32 and c.shape == (16,)
    assert np.all(np.diff(c.astype(np.float64)) > 0)
    assert c[0] == F32(-1.0) and c[7] == F32(0.0) and c[15] == F32(1.0)
    assert np.count_nonzero(c < 0) == 7 and np.count_nonzero(c > 0) == 8


def test_nf4_codebook_against_scipy_normal_quantiles():
    """Recompute the levels with scipy's ndtri (an independent routine) and
    check the forward CDF puts them at the evenly spaced probabilities."""
    from scipy.special import ndtr, ndtri
    delta = 1.0 - 0.5 * (1.0 / 30.0 + 1.0 / 32.0)
    top = ndtri(delta)
    pos = ndtri(np.linspace(delta, 0.5, 9)[:-1])
    neg = -ndtri(np.linspace(delta, 0.5, 8)[:-1])
    ref = np.sort(np.concatenate([pos, neg, [0.0]])) / top
    c = O.nf4_codebook()
    assert np.array_equal(ref.astype(F32), c)
    probs = ndtr(c[8:].astype(np.float64) * top)
    assert np.allclose(probs[::-1], np.linspace(delta, 0.5, 9)[:-1], atol=1e-6)


def test_nf4_codebook_golden_file():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "nf4_codebook.txt")) if not l.startswith("#")]
    stored = np.array([int(r[0], 16) for r in rows], dtype=np.uint32).view(F32)
    assert np.array_equal(stored, O.nf4_codebook())


def test_nf4_encode_is_nearest_level_bruteforce():
    W = SI.gaussian_weights(120, 64, 512, outlier_seed=121)
    codes, a = O.nf4_quantize(W, 64)
    c = O.nf4_codebook().astype(np.float64)
    blocks = W.reshape(-1, 64)
    x = (blocks / a[:, None]).astype(np.float64)  # the same fp32 x the rule sees
    d = np.abs(x[..., None] - c)
    best = d.argmin(-1)  # ties -> lower index (argmin returns the first)
    srt = np.sort(d, -1)
    near = (srt[..., 1] - srt[..., 0]) <= 2 * _f32_ulp(x) + 1e-12
    got = codes.reshape(-1, 64)
    assert not ((best != got) & ~near).any()
    # the block's absmax element encodes to an extreme level
    i = np.abs(blocks).argmax(1)
    ext = got[np.arange(len(i)), i]
    assert np.all((ext == 0) | (ext == 15))


def test_nf4_special_blocks():
    W = np.zeros((2, 128), dtype=F32)
    W[1, 64:] = np.tile(np.array([-0.5, 0.0, 0.5, 0.0], dtype=F32), 16)
    codes, a = O.nf4_quantize(W, 64)
    assert np.all(codes[0] == 7) and np.all(codes[1, :64] == 7)
    assert a[0] == 0 and a[2] == 0 and a[3] == F32(0.5)
    assert list(codes[1, 64:68]) == [0, 7, 15, 7]
    assert np.array_equal(O.nf4_exact(codes, a, 64), W.astype(np.float64))


def test_nf4_requantize_with_fixed_absmax_is_identity():
    W = SI.gaussian_weights(122, 32, 512)
    codes, a = O.nf4_quantize(W, 64)
    c = O.nf4_codebook()
    wh = (c[codes.reshape(-1, 64)] * a[:, None]).astype(F32)
    safe = np.where(a == 0, F32(1), a)
    x = wh / safe[:, None]
    again = np.searchsorted(O.nf4_midpoints(c), x, side="left")
    assert np.array_equal(again, codes.reshape(-1, 64))


# ---------------------------------------------------------------- double quant

def test_double_quant_values():
    rng = np.random.default_rng(130)
    a = np.abs(rng.standard_normal(1000)).astype(F32) * F32(0.05)
    q2, c2 = O.double_quant(a, 256)
    assert c2.shape == (4,) and q2.dtype == np.int8
    for b in range(4):
        seg = a[b * 256:(b + 1) * 256]
        assert c2[b] == seg.max() / F32(127)
        assert q2[b * 256 + int(seg.argmax())] == 127
        # brute force: each q2 is the nearest of 0..127 to a / c2 (ties excused)
        lv = np.arange(128) * np.float64(c2[b])
        d = np.abs(seg.astype(np.float64)[:, None] - lv)
        best = d.argmin(1)
        srt = np.sort(d, 1)
        near = (srt[:, 1] - srt[:, 0]) <= 4 * _f32_ulp(seg) + 1e-300
        assert not ((best != q2[b * 256:(b + 1) * 256]) & ~near).any()
    ah = O.double_dequant_absmax(q2, c2, 256)
    assert np.all(np.abs(ah.astype(np.float64) - a) <= 0.5 * np.repeat(c2, 256)[:1000] * (1 + 2.0 ** -20))
    zq, zc = O.double_quant(np.zeros(300, dtype=F32), 256)
    assert np.all(zq == 0) and np.all(zc == 0)


def test_double_quant_saving_closed_form():
    vals = dict(l.split() for l in open(os.path.join(GOLDEN, "dq_saving.txt")) if not l.startswith("#"))
    expect = float(vals["bits_per_param"])
    assert expect == 0.5 - (8 / 64 + 32 / (64 * 256))
    for shapes in (SI.LLAMA3_8B, SI.LLAMA3_70B, SI.QWEN15_110B):
        for n, k in shapes.values():
            assert O.dq_saving_bits_per_param(n, k) == expect
    # the byte counts the oracle actually produces agree with the formula
    W = SI.gaussian_weights(131, 64, 1024)
    codes, a = O.nf4_quantize(W, 64)
    q2, c2 = O.double_quant(a, 256)
    saved = a.nbytes - (q2.nbytes + c2.nbytes)
    assert 8.0 * saved / W.size == expect
    gb = float(vals["params_65b"]) * expect / 8
    assert abs(gb - float(vals["saving_bytes_65b_approx"])) < 0.05e9


# ---------------------------------------------------------------- matmuls

def _frac_bf16(bits):
    return [[Fraction(float(v)) for v in row] for row in O.bf16_to_f64(bits)]


def _frac_mat(a):
    return [[Fraction(float(v)) for v in row] for row in a]


def test_linear_fwd_matches_exact_rational_triple_loop():
    W = SI.gaussian_weights(140, 5, 128)
    q = O.quantize(W, "minmax", 4, 64)
    X = SI.bf16_normal(141, (3, 128))
    Y = O.linear_fwd(X, q["w_exact"])
    Xf, Wf = _frac_bf16(X), _frac_mat(q["w_exact"])
    for m in range(3):
        for n in range(5):
            exact = sum(Xf[m][k] * Wf[n][k] for k in range(128))
            assert abs(float(exact) - Y[m, n]) <= 1e-12 * max(1.0, abs(float(exact)))


def test_grid_matmul_is_exact_and_adjoint():
    """Grid weights and small-integer activations: every fp64 sum is exact, so
    forward and input-gradient must equal exact integer arithmetic, and
    <dY, X W^T> == <dY W, X> pins the transposes."""
    W = SI.grid_weights(142, 16, 256, 128, 4)
    q = O.quantize(W, "minmax", 4, 128)
    X = SI.bf16_small_ints(143, (4, 256))
    dY = SI.bf16_small_ints(144, (4, 16))
    Wi = (W.astype(np.float64) * 16).astype(np.int64)
    Xi = O.bf16_to_f64(X).astype(np.int64)
    dYi = O.bf16_to_f64(dY).astype(np.int64)
    Y = O.linear_fwd(X, q["w_exact"])
    dX = O.linear_bwd_dx(dY, q["w_exact"])
    Yi = np.array([[sum(int(Xi[m, k]) * int(Wi[n, k]) for k in range(256)) for n in range(16)] for m in range(4)])
    dXi = np.array([[sum(int(dYi[m, n]) * int(Wi[n, k]) for n in range(16)) for k in range(256)] for m in range(4)])
    assert np.array_equal(Y * 16, Yi.astype(np.float64))
    assert np.array_equal(dX * 16, dXi.astype(np.float64))
    assert (dYi * Yi).sum() == (dXi * Xi).sum()


def test_lora_zero_weight_is_pure_adapter_branch():
    rng_shapes = (3, 64, 8, 4)  # M, K, N, r
    M, K, N, r = rng_shapes
    W = np.zeros((N, K), dtype=F32)
    q = O.quantize(W, "nf4", double_quant_on=True)
    assert np.all(q["w_exact"] == 0)
    X = SI.bf16_normal(150, (M, K))
    A = SI.bf16_normal(151, (r, K), std=0.01)
    B = SI.bf16_normal(152, (N, r), std=0.01)
    for sigma in (1.0, 2.0):
        Y = O.lora_fwd(X, q["w_exact"], A, B, sigma)
        Xf, Af, Bf = _frac_bf16(X), _frac_bf16(A), _frac_bf16(B)
        for m in range(M):
            for n in range(N):
                t = [sum(Xf[m][k] * Af[j][k] for k in range(K)) for j in range(r)]
                exact = Fraction(sigma) * sum(t[j] * Bf[n][j] for j in range(r))
                assert abs(float(exact) - Y[m, n]) <= 1e-12 * max(1e-6, abs(float(exact)))


def test_channel_mix_equals_unsplit_layer():
    """Splitting the output channels into two sub-tensors of one format and
    scattering them back reproduces the unsplit layer exactly."""
    W = SI.gaussian_weights(160, 32, 256)
    X = SI.bf16_normal(161, (3, 256))
    rows4 = SI.channel_mask(162, 32)
    rows2 = np.setdiff1d(np.arange(32), rows4).astype(np.int32)
    full = O.quantize(W, "minmax", 4, 128)
    p4 = O.quantize(W[rows4], "minmax", 4, 128)
    p2 = O.quantize(W[rows2], "minmax", 4, 128)
    Y = O.channel_mix_fwd(X, [(rows4, p4["w_exact"]), (rows2, p2["w_exact"])])
    assert np.array_equal(Y, O.linear_fwd(X, full["w_exact"]))


def test_rel_errors_definition():
    ref = np.array([[3.0, 4.0]])
    fro, mx = O.rel_errors(ref + np.array([[0.0, 0.5]]), ref)
    assert fro == pytest.approx(0.1) and mx == pytest.approx(0.125)


# ---------------------------------------------------------------------------
# LoRA backward ("QLoRA技术在量化微调中的应用", section QLoRA技术原理): pinned to
# the forward by adjoint identities, and to brute force on a tiny case.
# ---------------------------------------------------------------------------


def _lora_case(seed, m=5, n=12, k=16, r=3):
    rng = np.random.default_rng(seed)
    X = SI.bf16_normal(seed + 1, (m, k))
    dY = SI.bf16_normal(seed + 2, (m, n))
    A = SI.bf16_normal(seed + 3, (r, k), std=0.5)
    B = SI.bf16_normal(seed + 4, (n, r), std=0.5)
    W = rng.standard_normal((n, k))
    return X, dY, W, A, B


def test_lora_bwd_adjoint_of_forward():
    """<dY, dY_dir> with the directional change of the forward equals the
    gradients paired with the direction.  The forward is bilinear in (A, B),
    so the central difference over +/- a direction is exact."""
    for sigma in (1.0, 2.0):
        X, dY, W, A, B = _lora_case(11)
        dX, dA, dB = O.lora_bwd(X, dY, W, A, B, sigma)
        rng = np.random.default_rng(5)
        dAd = rng.standard_normal(A.shape)
        dBd = rng.standard_normal(B.shape)
        Xf, dYf, Af, Bf = (O.bf16_to_f64(t) for t in (X, dY, A, B))

        def fwd(Xv, Av, Bv):
            return Xv @ W.T + sigma * (Xv @ Av.T) @ Bv.T

        diff = (fwd(Xf, Af + dAd, Bf + dBd) - fwd(Xf, Af - dAd, Bf - dBd)) / 2.0
        lhs = float(np.sum(dYf * diff))
        rhs = float(np.sum(dA * dAd) + np.sum(dB * dBd))
        assert abs(lhs - rhs) <= 1e-9 * max(1.0, abs(lhs))
        # dX: the forward is linear in X
        dXd = rng.standard_normal(Xf.shape)
        lhs = float(np.sum(dYf * (fwd(Xf + dXd, Af, Bf) - fwd(Xf, Af, Bf))))
        assert abs(lhs - float(np.sum(dX * dXd))) <= 1e-9 * max(1.0, abs(lhs))


def test_lora_bwd_brute_force_tiny():
    X, dY, W, A, B = _lora_case(23, m=3, n=4, k=5, r=2)
    sigma = 2.0
    dX, dA, dB = O.lora_bwd(X, dY, W, A, B, sigma)
    Xf, dYf, Af, Bf = (O.bf16_to_f64(t) for t in (X, dY, A, B))
    m, k = Xf.shape
    n, r = Bf.shape
    for a in range(m):
        for c in range(k):
            v = sum(dYf[a, i] * W[i, c] for i in range(n))
            v += sum(sigma * dYf[a, i] * Bf[i, j] * Af[j, c] for i in range(n) for j in range(r))
            assert abs(dX[a, c] - v) <= 1e-12 * max(1.0, abs(v))
    for j in range(r):
        for c in range(k):
            v = sum(sigma * dYf[a, i] * Bf[i, j] * Xf[a, c] for a in range(m) for i in range(n))
            assert abs(dA[j, c] - v) <= 1e-12 * max(1.0, abs(v))
    for i in range(n):
        for j in range(r):
            v = sum(sigma * dYf[a, i] * Xf[a, c] * Af[j, c] for a in range(m) for c in range(k))
            assert abs(dB[i, j] - v) <= 1e-12 * max(1.0, abs(v))


def test_grouped_input_gradient_is_the_adjoint_of_the_shared_forward():
    """Linears that read one X: <dX, X> equals the sum over the linears of
    <dY_i, X W_i^T> (exact on grid values, which pins the sum over the
    weights and every transpose), and sampled entries equal the brute-force
    sum over all the weights' rows."""
    X = SI.bf16_small_ints(150, (3, 256))
    Ws = [SI.grid_weights(151 + i, n, 256, 128, 4) for i, n in enumerate((16, 8, 24))]
    qs = [O.quantize(W, "minmax", 4, 128) for W in Ws]
    dYs = [SI.bf16_small_ints(160 + i, (3, W.shape[0])) for i, W in enumerate(Ws)]
    dX = O.linear_bwd_dx_grouped(dYs, [q["w_exact"] for q in qs])
    assert dX.shape == (3, 256)
    lhs = (dX * O.bf16_to_f64(X)).sum()
    rhs = sum((O.bf16_to_f64(d) * O.linear_fwd(X, q["w_exact"])).sum() for d, q in zip(dYs, qs))
    assert lhs == rhs
    for a in range(3):
        for c in range(0, 256, 37):
            v = sum(O.bf16_to_f64(d)[a, j] * q["w_exact"][j, c] for d, q in zip(dYs, qs) for j in range(d.shape[1]))
            assert dX[a, c] == v


# ---------------------------------------------------------------------------
# Exact ties.  Random inputs almost never put a quotient exactly on a
# half-integer or an NF4 value exactly on a midpoint, so the rounding rules
# are pinned on inputs built to sit on them (tests/tie_inputs.py); the
# expected integers come from exact rational arithmetic with the tie rule
# written out.
# ---------------------------------------------------------------------------
import tie_inputs as TI


def test_round_half_even_reference_rule():
    from fractions import Fraction as Fr
    got = [TI.round_half_even(Fr(t, 2)) for t in range(-7, 8)]
    assert got == [-4, -3, -2, -2, -2, -1, 0, 0, 0, 1, 2, 2, 2, 3, 4]
    assert TI.round_half_even(Fr(7, 3)) == 2 and TI.round_half_even(Fr(-7, 3)) == -2


def test_minmax_ties_literal_cases():
    """Literal expectations: with s = 2^-4, w = 2.5 s takes code 2 and 3.5 s
    code 4 (z = 0); -1.5 s takes -2 + z; a zero point at -lo/s = 2.5 is 2."""
    s = F32(1 / 16)
    W = np.zeros((2, 128), dtype=F32)
    W[0, :4] = [0.0, 15 * s, 2.5 * s, 3.5 * s]
    W[0, 4:] = 15 * s
    W[1, :4] = [-2.5 * s, 12.5 * s, -1.5 * s, 0.5 * s]
    W[1, 4:] = 0.0
    codes, sc, z = O.minmax_quantize(W, 4, 128)
    assert sc[0, 0] == s and sc[1, 0] == s
    assert z[0, 0] == 0 and list(codes[0, :4]) == [0, 15, 2, 4]
    assert z[1, 0] == 2                         # rne(2.5) = 2, not 3
    assert list(codes[1, :4]) == [0, 14, 0, 2]  # rne(-2.5)+2, rne(12.5)+2, rne(-1.5)+2, rne(0.5)+2


@pytest.mark.parametrize("bits,group", CASES)
def test_minmax_ties_round_half_to_even(bits, group):
    """Every code tie and every zero-point tie resolves to the even integer."""
    W, want = TI.minmax_tie_groups(bits, group)
    codes, s, z = O.minmax_quantize(W, bits, group)
    assert np.array_equal(s, want["scales"])
    assert np.array_equal(z, want["zeros"])
    assert np.array_equal(codes, want["codes"])


def test_double_quant_ties_round_half_to_even():
    a, want = TI.dq_tie_absmax()
    q2, c2 = O.double_quant(a, 256)
    assert np.array_equal(c2.view(np.uint32), want["absmax_scale"].view(np.uint32))
    assert np.array_equal(q2, want["absmax_q"])
    from fractions import Fraction as Fr
    # literal: a = 2.5 c2 -> 2, a = 3.5 c2 -> 4, a = 0.5 c2 -> 0
    lit = np.zeros(256, dtype=F32)
    lit[0] = F32(127 / 1024)
    lit[1:4] = [2.5 / 1024, 3.5 / 1024, 0.5 / 1024]
    q, c = O.double_quant(lit, 256)
    assert c[0] == F32(1 / 1024) and list(q[1:4]) == [2, 4, 0]
    assert TI.round_half_even(Fr(5, 2)) == 2


@pytest.mark.parametrize("scale_exp", [0, -3, 5])
def test_nf4_midpoint_ties_take_the_lower_code(scale_exp):
    """x exactly on midpoint m_i gives code i (a plain count of the midpoints
    strictly below x); one fp32 step above gives i + 1."""
    mids = O.nf4_midpoints(O.nf4_codebook())
    W, xs = TI.nf4_midpoint_blocks(mids, scale_exp)
    codes, a = O.nf4_quantize(W, 64)
    assert np.all(a == F32(2.0 ** scale_exp))
    for r in range(xs.shape[0]):
        for c in range(64):
            x = float(xs[r, c])
            want = 0
            for m in mids:
                if x > float(m):
                    want += 1
            assert codes[r, c] == want, (r, c, x, want, codes[r, c])
    for i, m in enumerate(mids):
        one = np.zeros((1, 64), dtype=F32)
        one[0, 0] = 1.0
        one[0, 1] = m
        one[0, 2] = np.nextafter(m, F32(2))
        c1, _ = O.nf4_quantize(one, 64)
        assert c1[0, 1] == i and c1[0, 2] == i + 1


@pytest.mark.parametrize("dq", [False, True])
def test_nf4_dequant_bf16_power_of_two_blocks(dq):
    """Blocks in {-a, 0, a} with a different a per block: the codes are 0, 7,
    15, double quantization is lossless on these a, and the dequantized bf16
    weight equals W exactly (checked against torch's conversion of W); an
    absmax read from the wrong block would change the value."""
    W = TI.nf4_power_of_two_blocks()
    ref = O.quantize(W, "nf4", double_quant_on=dq)
    assert set(np.unique(ref["codes"])) <= {0, 7, 15}
    expect = SI.to_bf16_bits(W)
    assert np.array_equal(O.bf16_to_f64(expect), W.astype(np.float64))
    assert np.array_equal(ref["w_bf16"], expect)
    ahat = ref["absmax_hat"] if dq else ref["absmax"]
    assert np.array_equal(O.nf4_dequant_bf16(ref["codes"], ahat, 64), expect)
    assert np.array_equal(ref["w_exact"], W.astype(np.float64))
    if dq:
        assert np.array_equal(ref["absmax_hat"], np.abs(W).reshape(-1, 64).max(1))


def test_minmax_dequant_bf16_per_group_scales():
    """Groups with a different power-of-two scale each: the dequantized bf16
    weight is W exactly; a scale or zero point read from another group would
    change it."""
    rng = np.random.default_rng(31)
    n, k, g = 6, 512, 128
    W = np.zeros((n, k), dtype=F32)
    for r in range(n):
        for j in range(k // g):
            z = int(rng.integers(0, 16))
            e = 3 + (r * (k // g) + j) % 9
            lv = rng.integers(0, 16, size=g)
            lv[0], lv[1] = 0, 15
            W[r, j * g:(j + 1) * g] = ((lv - z) * 2.0 ** -e).astype(F32)
    codes, s, z = O.minmax_quantize(W, 4, g)
    assert np.array_equal(O.minmax_dequant_bf16(codes, s, z, g), SI.to_bf16_bits(W))


# ---------------------------------------------------------------------------
# Format variants: compact MinMax metadata (fp16 scale rounded up, packed
# zero point) and double quantization with a per-tensor offset.
# ---------------------------------------------------------------------------

def _all_fp16_positive():
    """Every positive finite fp16 value, ascending, as fp64 (enumerated from
    the 16-bit patterns, independent of any rounding routine)."""
    bits = np.arange(1, 0x7C00, dtype=np.uint16)
    return bits.view(np.float16).astype(np.float64)


def test_fp16_round_up_is_smallest_fp16_not_below():
    table = _all_fp16_positive()
    rng = np.random.default_rng(300)
    s = np.concatenate([
        np.exp(rng.uniform(np.log(1e-9), np.log(6e4), 20000)).astype(F32),
        table[:2000].astype(F32), table[-2000:].astype(F32),                 # exact fp16 values stay
        np.nextafter(table[100:3000].astype(F32), F32(np.inf)),              # just above: next one up
        np.array([1e-30, 5.9604645e-08, 65504.0, 65505.0, 1e6], dtype=F32),
    ]).astype(F32)
    got = O.fp16_round_up(s).astype(np.float64)
    idx = np.searchsorted(table, s.astype(np.float64), side="left")
    want = np.where(idx < table.size, table[np.minimum(idx, table.size - 1)], 65504.0)
    assert np.array_equal(got, want)
    assert O.fp16_round_up(F32(1e-30)) == np.float16(2.0 ** -24)
    assert O.fp16_round_up(F32(1e6)) == np.float16(65504.0)


@pytest.mark.parametrize("bits,group", [(4, 128), (2, 64)])
def test_minmax_compact_codes_nearest_level_and_range(bits, group):
    """With the stored fp16 scale and zero point, every code is the nearest
    level (exhaustive fp64 search, near-ties excused); the stored scale is
    the fp32 scale rounded up, so Qmax * s covers the group's range."""
    qmax = (1 << bits) - 1
    W = np.concatenate([SI.gaussian_weights(310, 48, 4 * group, outlier_seed=311),
                        SI.student_t_weights(312, 16, 4 * group)])
    codes, s16, z = O.minmax_quantize_compact(W, bits, group)
    _, s32, _ = O.minmax_quantize(W, bits, group)
    s = s16.astype(np.float64)
    assert np.all(s >= s32) and np.all(s <= s32.astype(np.float64) * (1 + 2.0 ** -10))
    N, K = W.shape
    w = W.astype(np.float64).reshape(N, K // group, group)
    span = np.maximum(0, w.max(-1)) - np.minimum(0, w.min(-1))
    assert np.all(qmax * s >= span * (1 - 2.0 ** -22))
    levels = (np.arange(qmax + 1)[None, None, :] - z.astype(np.float64)[:, :, None]) * s[:, :, None]
    dist = np.abs(w[..., None] - levels[:, :, None, :])
    best = dist.argmin(-1)
    srt = np.sort(dist, -1)
    near = (srt[..., 1] - srt[..., 0]) <= 4 * _f32_ulp(w) + 1e-300
    assert not ((best != codes.reshape(best.shape)) & ~near).any()
    err = np.abs(w - (codes.reshape(w.shape).astype(np.float64) - z[:, :, None]) * s[:, :, None])
    assert np.all(err <= s[:, :, None] * (0.5 + 2.0 ** -18))


def test_minmax_compact_literal_and_power_of_two_cases():
    """A scale that fp16 holds exactly (2^-4) gives the fp32-metadata result
    bit for bit, ties included; s32 = 0.9/15 = 0.06 is stored as the fp16
    value just above it."""
    for bits, group in [(4, 128), (2, 64)]:
        W, want = TI.minmax_tie_groups(bits, group)
        codes, s16, z = O.minmax_quantize_compact(W, bits, group)
        assert np.all(s16 == np.float16(1 / 16))
        assert np.array_equal(codes, want["codes"]) and np.array_equal(z, want["zeros"])
    W = np.zeros((1, 128), dtype=F32)
    W[0, 0], W[0, 1] = F32(0.9), F32(-0.0)
    codes, s16, z = O.minmax_quantize_compact(W, 4, 128)
    table = _all_fp16_positive()
    s32 = F32(0.9) / F32(15)
    assert float(s16[0, 0]) == table[np.searchsorted(table, float(s32))] and float(s16[0, 0]) > float(s32)
    assert z[0, 0] == 0 and codes[0, 0] == 15 and codes[0, 1] == 0


@pytest.mark.parametrize("variant,bits", [("i4g128c", 4), ("i2g64c", 2)])
def test_compact_variant_arrays_and_bits_per_param(variant, bits):
    W = SI.gaussian_weights(320, 16, 1024)
    r = O.quantize_variant(W, variant)
    assert np.array_equal(O.unpack_codes(r["zeros_packed"], bits), r["zeros"])
    assert r["scales"].dtype == np.float16 and r["zeros_packed"].shape[1] * 8 == r["zeros"].shape[1] * bits
    expect = {"i4g128c": 4 + 16 / 128 + 4 / 128, "i2g64c": 2 + 16 / 64 + 2 / 64}[variant]
    assert expect == (4.15625 if bits == 4 else 2.28125)
    for n, k in list(SI.LLAMA3_8B.values()) + list(SI.QWEN15_110B.values()):
        assert O.variant_bits_per_param(variant, n, k) == expect
    got_bytes = r["packed"].nbytes + r["scales"].nbytes + r["zeros_packed"].nbytes
    assert 8.0 * got_bytes / W.size == expect
    assert np.array_equal(r["w_exact"], O.minmax_exact(r["codes"], r["scales"].astype(F32), r["zeros"],
                                                        128 if bits == 4 else 64))


def _tree_sum_recursive(a):
    """Brute-force reference of the adjacent-pair tree: split the zero-padded
    power-of-two range in halves, recursively, one fp32 addition per node."""
    n = 1
    while n < len(a):
        n *= 2
    v = [F32(x) for x in a] + [F32(0.0)] * (n - len(a))

    def rec(lo, hi):
        if hi - lo == 1:
            return v[lo]
        mid = (lo + hi) // 2
        return F32(rec(lo, mid) + rec(mid, hi))
    return rec(0, n) if n else F32(0.0)


def test_fp32_tree_sum():
    assert O.fp32_tree_sum(np.array([2.0 ** 24, 1, 1, 1], dtype=F32)) == F32(2.0 ** 24 + 2)  # a running sum gives 2^24
    rng = np.random.default_rng(330)
    for n in (1, 2, 3, 5, 8, 100, 255, 256, 257, 300):
        a = np.abs(rng.standard_normal(n)).astype(F32) * F32(10.0) ** rng.integers(-6, 6, n).astype(F32)
        assert O.fp32_tree_sum(a) == _tree_sum_recursive(a)
        ints = rng.integers(0, 1000, n).astype(F32)
        assert O.fp32_tree_sum(ints) == F32(int(ints.astype(np.int64).sum()))
    assert O.absmax_offset(np.array([1, 2, 3, 4], dtype=F32)) == F32(2.5)
    assert O.absmax_offset(np.full(1000, 0.375, dtype=F32)) == F32(0.375)


def test_double_quant_offset_ties_and_literal():
    a, want = TI.offset_tie_absmax()
    q2, c2, off = O.double_quant_offset(a, 256)
    assert off == F32(0.5) and np.all(c2 == F32(2.0 ** -10))
    assert np.array_equal(q2, want)
    assert (q2 < 0).any() and q2.min() == -127 and q2.max() == 127
    lit = np.array([0.5 + 127 / 1024, 0.5 - 127 / 1024, 0.5 + 2.5 / 1024, 0.5 - 2.5 / 1024], dtype=F32)
    q, c, o = O.double_quant_offset(np.tile(lit, 64), 256)
    assert o == F32(0.5) and list(q[:4]) == [127, -127, 2, -2]


def test_double_quant_offset_nearest_and_bound():
    rng = np.random.default_rng(340)
    a = (np.abs(rng.standard_normal(2000)) * 0.03 + 0.01).astype(F32)
    q2, c2, off = O.double_quant_offset(a, 256)
    q2p, c2p = O.double_quant(a, 256)
    assert np.all(c2.astype(np.float64) <= c2p.astype(np.float64) * (1 + 2.0 ** -20))
    d = (a - off).astype(np.float64)
    assert abs(float(off) - float(np.mean(a.astype(np.float64)))) <= 1e-6 * float(np.mean(a))
    for b in range(len(c2)):
        seg = d[b * 256:(b + 1) * 256]
        lv = np.arange(-127, 128) * np.float64(c2[b])
        dist = np.abs(seg[:, None] - lv)
        best = dist.argmin(1) - 127
        srt = np.sort(dist, 1)
        near = (srt[:, 1] - srt[:, 0]) <= 4 * _f32_ulp(a[b * 256:(b + 1) * 256]) + 1e-300
        assert not ((best != q2[b * 256:(b + 1) * 256]) & ~near).any()
        assert np.abs(q2[b * 256:(b + 1) * 256]).max() == 127
    ah = O.double_dequant_absmax_offset(q2, c2, off, 256).astype(np.float64)
    bound = 0.5 * np.repeat(c2, 256)[:2000] * (1 + 2.0 ** -20) + 2 * _f32_ulp(a)
    assert np.all(np.abs(ah - a) <= bound)


def test_nf4dqo_lossless_blocks_dequant_exact():
    """Block entries in {-A, 0, A} with absmax values that the offset
    variant reproduces exactly: the dequantized weight is W (fp32) exactly
    and its bf16 rounding equals torch's; the 4-bit codes equal those of
    plain NF4 (they come from the un-quantized absmax)."""
    a, _ = TI.offset_tie_absmax()
    # lossless: integer t, keep pairs; replace the half-integer ones by integers
    a = np.where(np.abs((a.astype(np.float64) - 0.5) * 1024 % 1) > 0, F32(0.5), a).astype(F32)
    rng = np.random.default_rng(350)
    blocks = np.zeros((a.size, 64), dtype=F32)
    for b in range(a.size):
        pat = rng.integers(-1, 2, 64)
        pat[rng.integers(0, 64)] = 1
        blocks[b] = pat * a[b]
    W = blocks.reshape(-1, 256)
    r = O.quantize_variant(W, "nf4dqo")
    assert np.array_equal(r["absmax_hat"], a)
    assert np.array_equal(r["w_exact"], W.astype(np.float64))
    assert np.array_equal(r["w_bf16"], SI.to_bf16_bits(W))
    assert np.array_equal(r["codes"], O.quantize(W, "nf4", double_quant_on=False)["codes"])
    assert r["absmax_scale"][-1] == F32(0.5) and r["absmax_scale"].shape == (a.size // 256 + 1,)


def test_nf4dqo_bits_per_param():
    """NF4 + double quantization costs 4.126953125 bit/param on these shapes
    (0.5 - 0.373046875 bits over the codes); the offset adds one fp32 per tensor."""
    for n, k in SI.LLAMA3_8B.values():
        assert O.variant_bits_per_param("nf4dqo", n, k) == 4.126953125 + 32.0 / (n * k)
