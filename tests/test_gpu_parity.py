"""GPU parity: the HIP path through the C ABI against the CPU oracle on the
same seeded inputs.

* quantize (codes, packed bytes, scales, zeros, absmax, absmax_q,
  absmax_scale) and dequantize (bf16) must be bit-exact;
* forward / input-gradient / LoRA must meet the matmul tolerance (relative
  Frobenius <= 5e-3, max-abs <= 2e-2 max|Y_ref| against fp64), and on inputs
  whose every partial sum is exact in fp32 they must equal bf16(exact) bit for
  bit, whichever kernel (GEMV or MFMA tile) runs.

Sizes span several tiles plus ragged tails (n not a multiple of the tile,
short K, m that is not a multiple of 16 or 128).
"""
import numpy as np
import pytest
import torch

import synth_inputs as SI
from oracle import lbq_oracle as O
from gpu_util import (DEV, assert_close, bf16_bits_host, check_quantized_equal, host,
                            to_dev_bf16, to_dev_f32)

pytestmark = pytest.mark.gpu

FORMATS = [
    ("minmax", 4, 128, False), ("minmax", 2, 64, False), ("minmax", 4, 64, False),
    ("minmax", 2, 128, False), ("nf4", 4, 64, False), ("nf4", 4, 64, True),
]
FMT_IDS = ["i4g128", "i2g64", "i4g64", "i2g128", "nf4", "nf4dq"]


@pytest.fixture(scope="module")
def L():
    import group_wise_minmax_amd as L
    assert torch.cuda.is_available()
    return L


def _quant_pair(L, W, fmt, bits, group, dq):
    qw = L.lbq_quantize(to_dev_f32(W), fmt, bits, group, dq)
    ref = O.quantize(W, fmt, bits, group, dq)
    return qw, ref


# ------------------------------------------------------------------ quantize


@pytest.mark.parametrize("fmtspec", FORMATS, ids=FMT_IDS)
@pytest.mark.parametrize("shape", [(256, 256), (3, 384), (1, 128), (37, 1280), (1000, 4096)])
def test_quantize_and_dequant_bitexact(L, fmtspec, shape):
    fmt, bits, group, dq = fmtspec
    n, k = shape
    W = SI.gaussian_weights(SI.seed_of(1, 0, 0) + n, n, k, outlier_seed=SI.seed_of(1, 0, 1) + n)
    qw, ref = _quant_pair(L, W, fmt, bits, group, dq)
    wb = L.lbq_dequant(qw)
    torch.cuda.synchronize()
    check_quantized_equal(qw, ref, fmt, dq)
    assert np.array_equal(bf16_bits_host(wb), ref["w_bf16"])


@pytest.mark.parametrize("fmtspec", FORMATS, ids=FMT_IDS)
def test_quantize_heavy_tailed_and_special_groups(L, fmtspec):
    fmt, bits, group, dq = fmtspec
    W = SI.student_t_weights(5010, 64, 1024)
    W[0, :] = 0.0                                   # all-zero rows / groups / blocks
    W[1, 5] = 3.0                                    # single nonzero groups
    W[2, :128] = -0.25                               # single-signed group
    W[3, 64:128] = np.tile(np.array([-0.5, 0.0, 0.5, 0.0], dtype=np.float32), 16)
    qw, ref = _quant_pair(L, W, fmt, bits, group, dq)
    wb = L.lbq_dequant(qw)
    torch.cuda.synchronize()
    check_quantized_equal(qw, ref, fmt, dq)
    assert np.array_equal(bf16_bits_host(wb), ref["w_bf16"])


@pytest.mark.parametrize("dq", [False, True], ids=["nf4", "nf4dq"])
def test_nf4_codes_at_midpoints_and_bucket_edges(L, dq):
    """Blocks whose absmax is 1 or 1/2 (so x = w / absmax is exact) put x on
    every NF4 midpoint (a tie takes the lower code), one ulp either side, and
    on every multiple of 1/32 in [-1, 1] with its neighbours: the codes, the
    absmax data and the dequantized weights equal the oracle's bit for bit."""
    mids = O.nf4_midpoints(O.nf4_codebook())
    steps = (-1.0 + np.arange(65, dtype=np.float64) / 32).astype(np.float32)
    pts = np.concatenate([mids, steps]).astype(np.float32)
    vals = np.concatenate([pts, np.nextafter(pts, np.float32(2)), np.nextafter(pts, np.float32(-2))])
    vals = np.clip(vals, np.float32(-1), np.float32(1)).astype(np.float32)
    nblk = -(-vals.size // 63)
    nblk += (-nblk) % 4                                # 4 blocks per row of 256
    body = np.resize(vals, nblk * 63).reshape(nblk, 63)
    blocks = np.concatenate([np.ones((nblk, 1), np.float32), body], axis=1)
    W = np.concatenate([blocks, blocks * np.float32(0.5)]).reshape(-1, 256).astype(np.float32)
    qw, ref = _quant_pair(L, W, "nf4", 4, 64, dq)
    wb = L.lbq_dequant(qw)
    torch.cuda.synchronize()
    check_quantized_equal(qw, ref, "nf4", dq)
    assert np.array_equal(bf16_bits_host(wb), ref["w_bf16"])


def test_quantize_config0_is_deterministic(L):
    """Single linear layer of 256x256, INT4 g128: two runs give identical bytes."""
    W = SI.gaussian_weights(SI.seed_of(0, 0, 0), 256, 256)
    a = L.lbq_quantize(to_dev_f32(W), "minmax", 4, 128)
    b = L.lbq_quantize(to_dev_f32(W), "minmax", 4, 128)
    torch.cuda.synchronize()
    assert torch.equal(a.packed, b.packed) and torch.equal(a.scales, b.scales)


# ------------------------------------------------------------------ forward

FWD_M = [1, 2, 3, 4, 5, 8, 16, 20, 33, 64, 65, 100, 130]


@pytest.mark.parametrize("fmtspec", FORMATS, ids=FMT_IDS)
@pytest.mark.parametrize("nk", [(300, 384), (256, 256), (1040, 1280)])
@pytest.mark.parametrize("m", FWD_M)
def test_forward_tolerance(L, fmtspec, nk, m):
    fmt, bits, group, dq = fmtspec
    n, k = nk
    W = SI.gaussian_weights(7000 + n, n, k, outlier_seed=7001 + n)
    X = SI.bf16_normal(7002 + m, (m, k))
    qw, ref = _quant_pair(L, W, fmt, bits, group, dq)
    Y = L.lbq_linear_fwd(to_dev_bf16(X), qw)
    torch.cuda.synchronize()
    assert_close(bf16_bits_host(Y), O.linear_fwd(X, ref["w_exact"]), what=f"{fmt}{bits}g{group} m={m}")


@pytest.mark.parametrize("fmtspec", FORMATS, ids=FMT_IDS)
@pytest.mark.parametrize("m", [1, 3, 4])
def test_forward_gemv_many_rows(L, fmtspec, m):
    """n = 4097 rows: many waves per launch and a ragged last row group."""
    fmt, bits, group, dq = fmtspec
    W = SI.gaussian_weights(7100, 4097, 512, outlier_seed=7101)
    X = SI.bf16_normal(7102, (m, 512))
    qw, ref = _quant_pair(L, W, fmt, bits, group, dq)
    Y = L.lbq_linear_fwd(to_dev_bf16(X), qw)
    torch.cuda.synchronize()
    assert_close(bf16_bits_host(Y), O.linear_fwd(X, ref["w_exact"]))


@pytest.mark.parametrize("fmtspec", FORMATS, ids=FMT_IDS)
@pytest.mark.parametrize("m", [2, 3, 4])
def test_forward_few_rows_match_single_rows(L, fmtspec, m):
    """2 <= m <= 4 streams the weight once for all rows of X; each output row
    equals, bit for bit, the m = 1 forward of that row (same per-row sums in
    the same order), and the oracle within the matmul tolerance.  n = 300
    leaves a ragged wave."""
    fmt, bits, group, dq = fmtspec
    n, k = 300, 2048
    W = SI.gaussian_weights(9700 + m, n, k, outlier_seed=9701)
    X = SI.bf16_normal(9702 + m, (m, k))
    qw, ref = _quant_pair(L, W, fmt, bits, group, dq)
    Xd = to_dev_bf16(X)
    Y = L.lbq_linear_fwd(Xd, qw)
    rows = [L.lbq_linear_fwd(Xd[i:i + 1].contiguous(), qw) for i in range(m)]
    torch.cuda.synchronize()
    for i in range(m):
        assert torch.equal(Y[i:i + 1].view(torch.int16), rows[i].view(torch.int16)), f"row {i}"
    assert_close(bf16_bits_host(Y), O.linear_fwd(X, ref["w_exact"]))


# Largest k whose m rows of x (m = 3..4) fit the multi-row GEMV's 64 KiB of
# LDS, per format: the next group up takes the small-batch MFMA kernel.
FEW_ROWS_KMAX = {"i4g128": 7680, "i2g64": 7936, "nf4dq": 4096}


@pytest.mark.parametrize("fid", list(FEW_ROWS_KMAX))
@pytest.mark.parametrize("above", [False, True], ids=["at_limit", "above_limit"])
def test_forward_few_rows_at_lds_limit(L, fid, above):
    """m = 4 at the longest rows the multi-row GEMV stages, and one group
    longer (the other kernel): both within the matmul tolerance of the oracle;
    at the limit each row also equals the m = 1 forward bit for bit."""
    fmt, bits, group, dq = FORMATS[FMT_IDS.index(fid)]
    m, n = 4, 200
    k = FEW_ROWS_KMAX[fid] + (group if above else 0)
    W = SI.gaussian_weights(9800 + k, n, k, outlier_seed=9801)
    X = SI.bf16_normal(9802 + k, (m, k))
    qw, ref = _quant_pair(L, W, fmt, bits, group, dq)
    Xd = to_dev_bf16(X)
    Y = L.lbq_linear_fwd(Xd, qw)
    rows = [L.lbq_linear_fwd(Xd[i:i + 1].contiguous(), qw) for i in range(m)] if not above else []
    torch.cuda.synchronize()
    for i, r in enumerate(rows):
        assert torch.equal(Y[i:i + 1].view(torch.int16), r.view(torch.int16)), f"row {i}"
    assert_close(bf16_bits_host(Y), O.linear_fwd(X, ref["w_exact"]), what=f"{fid} k={k}")


@pytest.mark.parametrize("fid", ["i4g128", "nf4dq"])
@pytest.mark.parametrize("m", [3, 4])
@pytest.mark.parametrize("n", [13056, 13120], ids=["gemv_rows", "mfma_rows"])
def test_forward_few_rows_tall_weight(L, fid, m, n):
    """At m = 3..4 a weight of more than 13056 rows (205 row tiles of 64, K
    within 16 chunks of 256) takes the small-batch MFMA kernel unsplit, one of
    13056 rows the multi-row GEMV: both within the matmul tolerance of the
    oracle, and on the GEMV side each row equals the m = 1 forward bit for
    bit."""
    fmt, bits, group, dq = FORMATS[FMT_IDS.index(fid)]
    k = 512
    W = SI.gaussian_weights(9900 + n + m, n, k, outlier_seed=9901)
    X = SI.bf16_normal(9902 + m, (m, k))
    qw, ref = _quant_pair(L, W, fmt, bits, group, dq)
    Xd = to_dev_bf16(X)
    Y = L.lbq_linear_fwd(Xd, qw)
    rows = [L.lbq_linear_fwd(Xd[i:i + 1].contiguous(), qw) for i in range(m)] if n == 13056 else []
    torch.cuda.synchronize()
    for i, r in enumerate(rows):
        assert torch.equal(Y[i:i + 1].view(torch.int16), r.view(torch.int16)), f"row {i}"
    assert_close(bf16_bits_host(Y), O.linear_fwd(X, ref["w_exact"]), what=f"{fid} n={n} m={m}")


@pytest.mark.parametrize("bits,group", [(4, 128), (2, 64), (4, 64), (2, 128)])
@pytest.mark.parametrize("m", [1, 2, 4, 7, 16, 130])
def test_forward_exact_on_grid_minmax(L, bits, group, m):
    """Lossless power-of-two-grid weights and integer activations: every
    partial sum is exact in fp32, so Y must equal bf16(X W^T) bit for bit."""
    n, k = 272, 512
    W = SI.grid_weights(7200, n, k, group, bits)
    X = SI.bf16_small_ints(7201 + m, (m, k))
    qw, ref = _quant_pair(L, W, "minmax", bits, group, False)
    assert np.array_equal(ref["w_exact"], W.astype(np.float64))
    Y = L.lbq_linear_fwd(to_dev_bf16(X), qw)
    torch.cuda.synchronize()
    exact = O.bf16_to_f64(X) @ W.astype(np.float64).T
    assert np.array_equal(bf16_bits_host(Y), O.bf16_bits(exact.astype(np.float32)))


@pytest.mark.parametrize("m", [1, 3, 16, 130])
def test_forward_exact_on_grid_nf4(L, m):
    """NF4 blocks holding only {-a, 0, +a} (a a power of two) encode to the
    levels -1, 0, +1 exactly, so again Y == bf16(exact)."""
    n, k = 200, 640
    rng = np.random.default_rng(7300)
    signs = rng.integers(-1, 2, size=(n * k // 64, 64)).astype(np.float64)
    signs[:, 0] = 1.0  # every block reaches +a, so its absmax is a
    a = 2.0 ** rng.integers(-6, -2, size=(n * k // 64, 1))
    W = (signs * a).astype(np.float32).reshape(n, k)
    X = SI.bf16_small_ints(7301 + m, (m, k))
    qw, ref = _quant_pair(L, W, "nf4", 4, 64, False)
    assert np.array_equal(ref["w_exact"], W.astype(np.float64))
    Y = L.lbq_linear_fwd(to_dev_bf16(X), qw)
    torch.cuda.synchronize()
    exact = O.bf16_to_f64(X) @ W.astype(np.float64).T
    assert np.array_equal(bf16_bits_host(Y), O.bf16_bits(exact.astype(np.float32)))


def test_forward_empty_batch_and_strided_output(L):
    W = SI.gaussian_weights(7400, 128, 256)
    qw = L.lbq_quantize(to_dev_f32(W), "minmax", 4, 128)
    X = torch.empty((0, 256), dtype=torch.bfloat16, device=DEV)
    Y = L.lbq_linear_fwd(X, qw)
    assert Y.shape == (0, 128)
    # ldy > n: only the first n columns are written
    Xb = SI.bf16_normal(7401, (5, 256))
    out = torch.full((5, 136), 7.0, dtype=torch.bfloat16, device=DEV)
    L.lbq_linear_fwd(to_dev_bf16(Xb), qw, out=out[:, :])
    torch.cuda.synchronize()
    ref = O.quantize(W, "minmax", 4, 128)
    assert_close(bf16_bits_host(out[:, :128]), O.linear_fwd(Xb, ref["w_exact"]))
    assert torch.all(out[:, 128:] == 7.0)


def test_forward_repeatable_bits(L):
    W = SI.gaussian_weights(7500, 1024, 1024)
    X = to_dev_bf16(SI.bf16_normal(7501, (300, 1024)))
    qw = L.lbq_quantize(to_dev_f32(W), "nf4", double_quant=True)
    a = L.lbq_linear_fwd(X, qw).clone()
    b = L.lbq_linear_fwd(X, qw)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


# Calls on different streams, each with its own workspace, share no state:
# the forwards of two weights launched in turn on two streams (so that they
# overlap) give the bits of the same calls run one after the other, for the
# GEMV (m = 1), the multi-row GEMV (2), the small-batch kernel with split K
# (16) and the GEMM with split K (300).
@pytest.mark.parametrize("m", [1, 2, 16, 300])
def test_forward_concurrent_streams(L, m):
    n, k, reps = 1024, 8192, 12
    qws = [L.lbq_quantize(to_dev_f32(SI.gaussian_weights(7600 + i, n, k)), "minmax", 4, 128) for i in range(2)]
    X = to_dev_bf16(SI.bf16_normal(7610 + m, (m, k)))
    ref = [L.lbq_linear_fwd(X, q).clone() for q in qws]
    wss = [torch.empty(max(16, L.lbq_linear_workspace_bytes(q, m)), dtype=torch.uint8, device=DEV) for q in qws]
    outs = [[torch.empty((m, n), dtype=torch.bfloat16, device=DEV) for _ in range(reps)] for _ in qws]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    for r in range(reps):
        for i in range(2):
            with torch.cuda.stream(streams[i]):
                L.lbq_linear_fwd(X, qws[i], out=outs[i][r], workspace=wss[i])
    torch.cuda.synchronize()
    for i in range(2):
        for r in range(reps):
            assert torch.equal(outs[i][r].view(torch.int16), ref[i].view(torch.int16)), (i, r)


# ------------------------------------------------------------------ backward


@pytest.mark.parametrize("fmtspec", FORMATS, ids=FMT_IDS)
@pytest.mark.parametrize("nk", [(264, 384), (1024, 1280)])
@pytest.mark.parametrize("m", [1, 5, 64, 130])
def test_bwd_dx_tolerance(L, fmtspec, nk, m):
    fmt, bits, group, dq = fmtspec
    n, k = nk
    W = SI.gaussian_weights(8000 + n, n, k, outlier_seed=8001 + n)
    dY = SI.bf16_normal(8002 + m, (m, n))
    qw, ref = _quant_pair(L, W, fmt, bits, group, dq)
    dX = L.lbq_linear_bwd_dx(to_dev_bf16(dY), qw)
    torch.cuda.synchronize()
    assert_close(bf16_bits_host(dX), O.linear_bwd_dx(dY, ref["w_exact"]), what=f"bwd {fmt} m={m}")


# The 256x256 tiles (picked for m = 4096 and 4096 output columns) run their
# K loop in two phases; few K-steps exercise its first and last stages.
@pytest.mark.parametrize("fid,kk", [("nf4dq", 64), ("nf4dq", 192), ("i4g128", 128), ("i4g128", 384),
                                    ("i2g64", 64)])
def test_gemm_large_tiles_few_k_steps(L, fid, kk):
    """Forward Y = X . W^T with k = kk and input gradient dX = dY . W with
    n = kk (the reduction of each runs over one to six 64-wide steps), both
    with 4096 x 4096 outputs; 64 sampled rows against the oracle."""
    fmt, bits, group, dq = FORMATS[FMT_IDS.index(fid)]
    m = 4096
    rows = np.sort(np.random.default_rng(9950 + kk).choice(m, 64, replace=False))
    # forward: W [4096][kk]
    W = SI.gaussian_weights(9951 + kk, 4096, kk, outlier_seed=9952)
    X = SI.bf16_normal(9953 + kk, (m, kk))
    qw, ref = _quant_pair(L, W, fmt, bits, group, dq)
    Y = L.lbq_linear_fwd(to_dev_bf16(X), qw)
    torch.cuda.synchronize()
    assert_close(bf16_bits_host(Y)[rows], O.linear_fwd(X[rows], ref["w_exact"]), what=f"fwd {fid} k={kk}")
    # input gradient: W [kk][4096]
    W2 = SI.gaussian_weights(9954 + kk, kk, 4096, outlier_seed=9955)
    dY = SI.bf16_normal(9956 + kk, (m, kk))
    qw2, ref2 = _quant_pair(L, W2, fmt, bits, group, dq)
    dX = L.lbq_linear_bwd_dx(to_dev_bf16(dY), qw2)
    torch.cuda.synchronize()
    assert_close(bf16_bits_host(dX)[rows], O.linear_bwd_dx(dY[rows], ref2["w_exact"]), what=f"bwd {fid} n={kk}")


@pytest.mark.parametrize("fid", ["i4g128", "i2g64", "nf4dq"])
@pytest.mark.parametrize("m", [3, 130, 300])
def test_bwd_dx_grouped(L, fid, m):
    """dX = sum_i dY_i . deq(W_i) for weights that share X, in one launch:
    bit for bit the input gradient of the weights stacked along n (the 320-
    and 64-row weights end on 64-row stage boundaries, the 200-row weight in
    a partial stage; NF4+DQ's 256-block groups do not straddle weights), and
    within the matmul tolerance of the oracle."""
    fmt, bits, group, dq = FORMATS[FMT_IDS.index(fid)]
    k, ns = 1280, (320, 64, 200)
    Ws = [SI.gaussian_weights(9600 + i, n, k, outlier_seed=9610 + i) for i, n in enumerate(ns)]
    pairs = [_quant_pair(L, W, fmt, bits, group, dq) for W in Ws]
    dYs = [SI.bf16_normal(9620 + 10 * i + m, (m, n)) for i, n in enumerate(ns)]
    dX = L.lbq_linear_bwd_dx_grouped([to_dev_bf16(d) for d in dYs], [p[0] for p in pairs])
    q_all = L.lbq_quantize(to_dev_f32(np.concatenate(Ws)), fmt, bits, group, dq)
    dX_all = L.lbq_linear_bwd_dx(to_dev_bf16(np.concatenate(dYs, axis=1)), q_all)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits_host(dX), bf16_bits_host(dX_all)), f"{fid} m={m}: grouped != stacked"
    assert_close(bf16_bits_host(dX), O.linear_bwd_dx_grouped(dYs, [p[1]["w_exact"] for p in pairs]),
                 what=f"grouped bwd {fid} m={m}")


@pytest.mark.parametrize("fid", ["i4g64", "nf4"])
def test_bwd_dx_grouped_ragged_and_single(L, fid):
    """Weights whose row counts are not multiples of 64 (each ends in a
    partial stage) against the oracle; a set of one equals lbq_linear_bwd_dx
    bit for bit."""
    fmt, bits, group, dq = FORMATS[FMT_IDS.index(fid)]
    k, m, ns = 640, 130, (136, 8, 72)
    pairs = [_quant_pair(L, SI.gaussian_weights(9640 + i, n, k, outlier_seed=9650 + i), fmt, bits, group, dq)
             for i, n in enumerate(ns)]
    dYs = [SI.bf16_normal(9660 + i, (m, n)) for i, n in enumerate(ns)]
    dYd = [to_dev_bf16(d) for d in dYs]
    dX = L.lbq_linear_bwd_dx_grouped(dYd, [p[0] for p in pairs])
    one = L.lbq_linear_bwd_dx_grouped(dYd[:1], [pairs[0][0]])
    single = L.lbq_linear_bwd_dx(dYd[0], pairs[0][0])
    torch.cuda.synchronize()
    assert_close(bf16_bits_host(dX), O.linear_bwd_dx_grouped(dYs, [p[1]["w_exact"] for p in pairs]),
                 what=f"grouped bwd {fid} ragged")
    assert np.array_equal(bf16_bits_host(one), bf16_bits_host(single))


@pytest.mark.parametrize("fid", ["i4g128", "i2g64", "i4g64"])
def test_bwd_dx_column_cut(L, fid):
    """An input gradient whose 256x256 tiles leave the last round partly
    empty (k = 4608 at m = 4000: 18 x 16 = 288 tiles) runs as two launches,
    columns [0, 4096) on 256x256 tiles and the rest on 128x128 tiles.  The
    same weight without its first 512 columns (k = 4096: one round of
    256x256 tiles) must give the same bits for the shared columns, and 48
    sampled rows match the oracle."""
    fmt, bits, group, dq = FORMATS[FMT_IDS.index(fid)]
    m, n, k = 4000, 256, 4608
    rows = np.sort(np.random.default_rng(9490).choice(m, 48, replace=False))
    W = SI.gaussian_weights(9491, n, k, outlier_seed=9492)
    dY = SI.bf16_normal(9493, (m, n))
    qw, ref = _quant_pair(L, W, fmt, bits, group, dq)
    qw2, _ = _quant_pair(L, np.ascontiguousarray(W[:, 512:]), fmt, bits, group, dq)
    dYd = to_dev_bf16(dY)
    dX = L.lbq_linear_bwd_dx(dYd, qw)
    dX2 = L.lbq_linear_bwd_dx(dYd, qw2)
    torch.cuda.synchronize()
    got = bf16_bits_host(dX)
    assert np.array_equal(got[:, 512:], bf16_bits_host(dX2)), f"{fid}: the cut changed bits"
    assert_close(got[rows], O.linear_bwd_dx(dY[rows], ref["w_exact"]), what=f"{fid} cut bwd")


@pytest.mark.parametrize("bits,group", [(4, 128), (2, 64)])
@pytest.mark.parametrize("m", [3, 130])
def test_bwd_dx_exact_on_grid(L, bits, group, m):
    n, k = 136, 640
    W = SI.grid_weights(8100, n, k, group, bits)
    dY = SI.bf16_small_ints(8101 + m, (m, n))
    qw, _ = _quant_pair(L, W, "minmax", bits, group, False)
    dX = L.lbq_linear_bwd_dx(to_dev_bf16(dY), qw)
    torch.cuda.synchronize()
    exact = O.bf16_to_f64(dY) @ W.astype(np.float64)
    assert np.array_equal(bf16_bits_host(dX), O.bf16_bits(exact.astype(np.float32)))


# ------------------------------------------------------------------ LoRA


@pytest.mark.parametrize("fmtspec", [FORMATS[0], FORMATS[5]], ids=["i4g128", "nf4dq"])
@pytest.mark.parametrize("m", [1, 4, 40, 130])
@pytest.mark.parametrize("r", [16, 8, 40])
def test_lora_tolerance(L, fmtspec, m, r):
    fmt, bits, group, dq = fmtspec
    n, k = 320, 512
    W = SI.gaussian_weights(9000, n, k)
    X = SI.bf16_normal(9001 + m, (m, k))
    A = SI.bf16_normal(9002, (r, k), std=0.01)
    B = SI.bf16_normal(9003, (n, r), std=0.01)
    qw, ref = _quant_pair(L, W, fmt, bits, group, dq)
    Y = L.lbq_lora_fwd(to_dev_bf16(X), qw, to_dev_bf16(A), to_dev_bf16(B), 16.0 / r)
    torch.cuda.synchronize()
    assert_close(bf16_bits_host(Y), O.lora_fwd(X, ref["w_exact"], A, B, 16.0 / r))


@pytest.mark.parametrize("m", [2, 130])
@pytest.mark.parametrize("sigma", [1.0, 2.0])
def test_lora_branch_alone_on_zero_weight(L, m, sigma):
    """W == 0 quantizes to exact zeros, leaving only sigma (X A^T) B^T: a wrong
    sigma or a transposed adapter cannot hide behind the base matmul."""
    n, k, r = 256, 384, 16
    W = np.zeros((n, k), dtype=np.float32)
    X = SI.bf16_normal(9100 + m, (m, k))
    A = SI.bf16_normal(9101, (r, k), std=0.01)
    B = SI.bf16_normal(9102, (n, r), std=0.01)
    qw, ref = _quant_pair(L, W, "nf4", 4, 64, True)
    Y = L.lbq_lora_fwd(to_dev_bf16(X), qw, to_dev_bf16(A), to_dev_bf16(B), sigma)
    torch.cuda.synchronize()
    assert_close(bf16_bits_host(Y), O.lora_fwd(X, ref["w_exact"], A, B, sigma))


def assert_close_f32(got: torch.Tensor, ref: np.ndarray, what=""):
    """fp32 adapter gradients against the fp64 oracle, to the matmul tolerance."""
    fro, mx = O.rel_errors(host(got).astype(np.float64), ref)
    assert fro <= 5e-3 and mx <= 2e-2, f"{what}: rel_fro={fro:.3e} max_rel={mx:.3e}"


@pytest.mark.parametrize("fmtspec", [FORMATS[0], FORMATS[5]], ids=["i4g128", "nf4dq"])
@pytest.mark.parametrize("m", [1, 5, 64, 130, 300])
@pytest.mark.parametrize("r", [16, 8, 40, 64])
def test_lora_bwd_tolerance(L, fmtspec, m, r):
    fmt, bits, group, dq = fmtspec
    n, k = 320, 512
    W = SI.gaussian_weights(9300, n, k)
    X = SI.bf16_normal(9301 + m, (m, k))
    dY = SI.bf16_normal(9302 + m, (m, n))
    A = SI.bf16_normal(9303, (r, k), std=0.01)
    B = SI.bf16_normal(9304, (n, r), std=0.01)
    sigma = 16.0 / r
    qw, ref = _quant_pair(L, W, fmt, bits, group, dq)
    dX, dA, dB = L.lbq_lora_bwd(to_dev_bf16(X), to_dev_bf16(dY), qw, to_dev_bf16(A), to_dev_bf16(B), sigma)
    torch.cuda.synchronize()
    rX, rA, rB = O.lora_bwd(X, dY, ref["w_exact"], A, B, sigma)
    assert_close(bf16_bits_host(dX), rX, what=f"lora bwd dX {fmt} m={m} r={r}")
    assert_close_f32(dA, rA, what=f"lora bwd dA m={m} r={r}")
    assert_close_f32(dB, rB, what=f"lora bwd dB m={m} r={r}")


@pytest.mark.parametrize("m", [3, 130])
@pytest.mark.parametrize("sigma", [1.0, 2.0])
def test_lora_bwd_on_zero_weight(L, m, sigma):
    """W == 0 leaves dX = sigma (dY B) A alone: the adapter term of the input
    gradient is checked without the base product to hide a wrong sigma or a
    transposed factor."""
    n, k, r = 256, 384, 16
    W = np.zeros((n, k), dtype=np.float32)
    X = SI.bf16_normal(9310 + m, (m, k))
    dY = SI.bf16_normal(9311 + m, (m, n))
    A = SI.bf16_normal(9312, (r, k), std=0.05)
    B = SI.bf16_normal(9313, (n, r), std=0.05)
    qw, ref = _quant_pair(L, W, "nf4", 4, 64, True)
    dX, dA, dB = L.lbq_lora_bwd(to_dev_bf16(X), to_dev_bf16(dY), qw, to_dev_bf16(A), to_dev_bf16(B), sigma)
    torch.cuda.synchronize()
    rX, rA, rB = O.lora_bwd(X, dY, ref["w_exact"], A, B, sigma)
    assert np.abs(ref["w_exact"]).max() == 0.0
    assert_close(bf16_bits_host(dX), rX, what=f"zero-W lora dX sigma={sigma}")
    assert_close_f32(dA, rA, what="zero-W dA")
    assert_close_f32(dB, rB, what="zero-W dB")


def test_lora_bwd_empty_batch_zeros_adapter_grads(L):
    n, k, r = 128, 256, 16
    qw, _ = _quant_pair(L, SI.gaussian_weights(9320, n, k), "minmax", 4, 128, False)
    X = torch.empty((0, k), dtype=torch.bfloat16, device=DEV)
    dY = torch.empty((0, n), dtype=torch.bfloat16, device=DEV)
    A = to_dev_bf16(SI.bf16_normal(9321, (r, k)))
    B = to_dev_bf16(SI.bf16_normal(9322, (n, r)))
    dA = torch.full((r, k), 7.0, dtype=torch.float32, device=DEV)
    dB = torch.full((n, r), 7.0, dtype=torch.float32, device=DEV)
    _, dA, dB = L.lbq_lora_bwd(X, dY, qw, A, B, 1.0, dA=dA, dB=dB)
    torch.cuda.synchronize()
    assert not host(dA).any() and not host(dB).any()


def test_lora_bwd_deterministic(L):
    n, k, r, m = 512, 1024, 16, 700
    qw, _ = _quant_pair(L, SI.gaussian_weights(9330, n, k), "nf4", 4, 64, True)
    X = to_dev_bf16(SI.bf16_normal(9331, (m, k)))
    dY = to_dev_bf16(SI.bf16_normal(9332, (m, n)))
    A = to_dev_bf16(SI.bf16_normal(9333, (r, k), std=0.01))
    B = to_dev_bf16(SI.bf16_normal(9334, (n, r), std=0.01))
    first = [t.clone() for t in L.lbq_lora_bwd(X, dY, qw, A, B, 1.0)]
    for _ in range(2):
        again = L.lbq_lora_bwd(X, dY, qw, A, B, 1.0)
        for a, b in zip(first, again):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))


def test_lora_autograd_layer(L):
    """LbqLoraLinear through torch.autograd: forward, dX, dA and dB against the
    oracle (X of shape [2, 3, k]: leading dimensions flatten to m = 6); a
    fresh layer (B = 0) reproduces the frozen forward."""
    n, k, r, alpha = 256, 512, 16, 32.0
    qw, ref = _quant_pair(L, SI.gaussian_weights(9600, n, k), "nf4", 4, 64, True)
    X = SI.bf16_normal(9601, (2, 3, k))
    dY = SI.bf16_normal(9602, (2, 3, n))
    A = SI.bf16_normal(9603, (r, k), std=0.01)
    B = SI.bf16_normal(9604, (n, r), std=0.01)
    fresh = L.LbqLoraLinear(qw, r=r, lora_alpha=alpha)
    Xd = to_dev_bf16(X)
    assert torch.equal(fresh(Xd).reshape(6, n).view(torch.int16), L.lbq_linear_fwd(Xd.reshape(6, k), qw).view(torch.int16))
    layer = L.LbqLoraLinear(qw, r=r, lora_alpha=alpha)
    with torch.no_grad():
        layer.A.copy_(to_dev_bf16(A).float())
        layer.B.copy_(to_dev_bf16(B).float())
    Xg = to_dev_bf16(X).requires_grad_(True)
    Y = layer(Xg)
    Y.backward(to_dev_bf16(dY))
    torch.cuda.synchronize()
    sigma = alpha / r
    Xf, dYf = X.reshape(6, k), dY.reshape(6, n)
    assert_close(bf16_bits_host(Y.detach().reshape(6, n)), O.lora_fwd(Xf, ref["w_exact"], A, B, sigma), what="autograd fwd")
    rX, rA, rB = O.lora_bwd(Xf, dYf, ref["w_exact"], A, B, sigma)
    assert Xg.grad.dtype == torch.bfloat16 and layer.A.grad.dtype == torch.float32
    assert_close(bf16_bits_host(Xg.grad.reshape(6, k)), rX, what="autograd dX")
    assert_close_f32(layer.A.grad, rA, what="autograd dA")
    assert_close_f32(layer.B.grad, rB, what="autograd dB")


# ------------------------------------------------------------------ mixed precision


@pytest.mark.parametrize("m", [1, 2, 3, 4, 16, 130])
def test_channel_mix_scatter(L, m):
    """25% of the output channels in INT4 g128, 75% in INT2 g64, each a
    separate quantized tensor whose out_rows scatter into one Y."""
    n, k = 512, 384
    W = SI.gaussian_weights(9200, n, k, outlier_seed=9201)
    rows4 = SI.channel_mask(9202, n)
    rows2 = np.setdiff1d(np.arange(n), rows4).astype(np.int32)
    X = SI.bf16_normal(9203 + m, (m, k))
    q4, r4 = _quant_pair(L, W[rows4], "minmax", 4, 128, False)
    q2, r2 = _quant_pair(L, W[rows2], "minmax", 2, 64, False)
    q4.out_rows = torch.from_numpy(rows4).to(DEV)
    q2.out_rows = torch.from_numpy(rows2).to(DEV)
    Y = torch.zeros((m, n), dtype=torch.bfloat16, device=DEV)
    Xd = to_dev_bf16(X)
    L.lbq_linear_fwd(Xd, q4, out=Y)
    L.lbq_linear_fwd(Xd, q2, out=Y)
    Yg = torch.zeros((m, n), dtype=torch.bfloat16, device=DEV)
    L.lbq_linear_fwd_grouped(Xd, [q4, q2], outs=[Yg, Yg])  # both row sets in one call
    torch.cuda.synchronize()
    ref = O.channel_mix_fwd(X, [(rows4, r4["w_exact"]), (rows2, r2["w_exact"])])
    assert_close(bf16_bits_host(Y), ref)
    assert np.array_equal(bf16_bits_host(Yg), bf16_bits_host(Y))


# ------------------------------------------------------------------ GEMM K split

# A GEMM whose 256x256 tiles fill at most half the chip splits K into ranges
# of at least 3200 codes (512 for m <= 256 when it fills at most an eighth of
# the chip): k = 8192 splits at any m.
SPLIT_K = 8192


@pytest.mark.parametrize("fmtspec", FORMATS, ids=FMT_IDS)
@pytest.mark.parametrize("n,m", [(518, 100), (1024, 257)])
def test_gemm_split_k(L, fmtspec, n, m):
    """m > 64 with few output tiles and long K: the GEMM splits K over
    workgroups (whole 1024-code blocks, so every metadata batch starts in its
    range) and a second kernel sums their fp32 partials.  That forward and the
    unsplit GEMM (an empty workspace) both meet the matmul tolerance; n = 518
    takes the partials' scalar stores."""
    fmt, bits, group, dq = fmtspec
    k = SPLIT_K
    W = SI.gaussian_weights(9600 + n, n, k, outlier_seed=9601)
    X = SI.bf16_normal(9602 + m, (m, k))
    qw, ref = _quant_pair(L, W, fmt, bits, group, dq)
    assert L.lbq_linear_workspace_bytes(qw, m) > 0  # the split is on
    Xd = to_dev_bf16(X)
    Ys = L.lbq_linear_fwd(Xd, qw)
    Yu = L.lbq_linear_fwd(Xd, qw, workspace=torch.empty(0, dtype=torch.uint8, device=DEV))
    torch.cuda.synchronize()
    Yref = O.linear_fwd(X, ref["w_exact"])
    assert_close(bf16_bits_host(Ys), Yref, what=f"{fmt}{bits}g{group} split n={n} m={m}")
    assert_close(bf16_bits_host(Yu), Yref, what=f"{fmt}{bits}g{group} unsplit n={n} m={m}")


@pytest.mark.parametrize("fmtspec", FORMATS, ids=FMT_IDS)
@pytest.mark.parametrize("n,k,m", [(520, 2048, 130), (300, 1536, 65), (4096, 4096, 256)])
def test_gemm_split_k_short_k(L, fmtspec, n, k, m):
    """65 <= m <= 256: ranges down to 512 codes (3 and 4 of them here, 8 at
    the 8B o shape), against the oracle, and equal run to run."""
    fmt, bits, group, dq = fmtspec
    W = SI.gaussian_weights(9670 + n, n, k, outlier_seed=9671)
    X = SI.bf16_normal(9672 + m, (m, k))
    qw, ref = _quant_pair(L, W, fmt, bits, group, dq)
    assert L.lbq_linear_workspace_bytes(qw, m) > 0  # the split is on
    Xd = to_dev_bf16(X)
    Y = L.lbq_linear_fwd(Xd, qw)
    Y2 = L.lbq_linear_fwd(Xd, qw)
    torch.cuda.synchronize()
    assert torch.equal(Y.view(torch.int16), Y2.view(torch.int16))
    assert_close(bf16_bits_host(Y), O.linear_fwd(X, ref["w_exact"]), what=f"{fmt}{bits}g{group} n={n} k={k} m={m}")


def test_gemm_split_k_channel_mix_scatter(L):
    """The channel-mixed layer's two row sets at m = 130 and k = 8192: both
    GEMMs split K and the reduce scatters through out_rows; one grouped call
    equals the two single calls bit for bit."""
    m, n, k = 130, 512, SPLIT_K
    W = SI.gaussian_weights(9650, n, k, outlier_seed=9651)
    rows4 = SI.channel_mask(9652, n)
    rows2 = np.setdiff1d(np.arange(n), rows4).astype(np.int32)
    X = SI.bf16_normal(9653, (m, k))
    q4, r4 = _quant_pair(L, W[rows4], "minmax", 4, 128, False)
    q2, r2 = _quant_pair(L, W[rows2], "minmax", 2, 64, False)
    q4.out_rows = torch.from_numpy(rows4).to(DEV)
    q2.out_rows = torch.from_numpy(rows2).to(DEV)
    assert L.lbq_linear_workspace_bytes(q4, m) > 0 and L.lbq_linear_workspace_bytes(q2, m) > 0
    Xd = to_dev_bf16(X)
    Y = torch.zeros((m, n), dtype=torch.bfloat16, device=DEV)
    L.lbq_linear_fwd(Xd, q4, out=Y)
    L.lbq_linear_fwd(Xd, q2, out=Y)
    Yg = torch.zeros((m, n), dtype=torch.bfloat16, device=DEV)
    L.lbq_linear_fwd_grouped(Xd, [q4, q2], outs=[Yg, Yg])
    torch.cuda.synchronize()
    ref = O.channel_mix_fwd(X, [(rows4, r4["w_exact"]), (rows2, r2["w_exact"])])
    assert_close(bf16_bits_host(Y), ref)
    assert np.array_equal(bf16_bits_host(Yg), bf16_bits_host(Y))


@pytest.mark.parametrize("fmtspec", [FORMATS[0], FORMATS[5]], ids=["i4g128", "nf4dq"])
def test_gemm_split_k_lora(L, fmtspec):
    """LoRA forward through a GEMM that splits K: the adapter slab is added
    once, by the range that starts at k = 0."""
    fmt, bits, group, dq = fmtspec
    m, n, k, r = 130, 512, SPLIT_K, 16
    W = SI.gaussian_weights(9660, n, k)
    X = SI.bf16_normal(9661, (m, k))
    A = SI.bf16_normal(9662, (r, k), std=0.01)
    B = SI.bf16_normal(9663, (n, r), std=0.01)
    qw, ref = _quant_pair(L, W, fmt, bits, group, dq)
    assert L.lbq_linear_workspace_bytes(qw, m) > 0
    Y = L.lbq_lora_fwd(to_dev_bf16(X), qw, to_dev_bf16(A), to_dev_bf16(B), 1.0)
    torch.cuda.synchronize()
    assert_close(bf16_bits_host(Y), O.lora_fwd(X, ref["w_exact"], A, B, 1.0))


@pytest.mark.parametrize("fmtspec", FORMATS, ids=FMT_IDS)
def test_forward_gemv_long_rows(L, fmtspec):
    """k = 36864: the arranged x no longer fits the GEMV's LDS budget, so x is
    read from global memory with every step."""
    fmt, bits, group, dq = fmtspec
    n, k = 72, 36864
    W = SI.gaussian_weights(9300, n, k, outlier_seed=9301)
    X = SI.bf16_normal(9302, (1, k))
    qw, ref = _quant_pair(L, W, fmt, bits, group, dq)
    Y = L.lbq_linear_fwd(to_dev_bf16(X), qw)
    torch.cuda.synchronize()
    assert_close(bf16_bits_host(Y), O.linear_fwd(X, ref["w_exact"]), what=f"{fmt}{bits}g{group} long rows")


# ------------------------------------------------------------------ grouped forward (shared X)

GROUP_SETS = {
    "three_i4g128": [FORMATS[0]] * 3,
    "mixed_kinds": [FORMATS[0], FORMATS[1], FORMATS[5], FORMATS[0]],
    # the channel-mixed layer's two formats only (one launch at m = 1)
    "channel_mix": [FORMATS[0], FORMATS[1], FORMATS[1], FORMATS[0]],
}


@pytest.mark.parametrize("name", list(GROUP_SETS))
@pytest.mark.parametrize("k", [1280, 12288])
@pytest.mark.parametrize("m", [1, 2, 3, 4, 16, 40, 57, 130, 300])
def test_grouped_fwd_matches_single(L, name, k, m):
    """Weights sharing X in one call: each output equals the single-weight
    forward bit for bit (same kernels, same per-row order) and the oracle
    within the matmul tolerance.  Ragged n; at m = 1 same-kind weights share
    one launch and the mixed set needs three, at every m (the channel-mix set
    one, up to m = 64): the GEMVs, the multi-row GEMV, the small-batch kernel (each weight keeping its own K split, so the sums run
    in the same order) and the GEMM, which lays the weights' column tiles
    side by side."""
    specs = GROUP_SETS[name]
    ns = [300, 64, 520, 130][:len(specs)]
    X = SI.bf16_normal(9400 + m, (m, k))
    qws, refs = [], []
    for i, ((fmt, bits, group, dq), n) in enumerate(zip(specs, ns)):
        qw, ref = _quant_pair(L, SI.gaussian_weights(9410 + i, n, k, outlier_seed=9420 + i), fmt, bits, group, dq)
        qws.append(qw)
        refs.append(ref)
    Xd = to_dev_bf16(X)
    Ys = L.lbq_linear_fwd_grouped(Xd, qws)
    singles = [L.lbq_linear_fwd(Xd, q) for q in qws]
    torch.cuda.synchronize()
    for i, (Y, Y1, ref) in enumerate(zip(Ys, singles, refs)):
        assert np.array_equal(bf16_bits_host(Y), bf16_bits_host(Y1)), f"{name} weight {i}: grouped != single"
        assert_close(bf16_bits_host(Y), O.linear_fwd(X, ref["w_exact"]), what=f"{name} weight {i} m={m}")


@pytest.mark.parametrize("k", [1280, 8192], ids=["k1280", "k8192_split"])
@pytest.mark.parametrize("m", [130, 300])
def test_grouped_mixed_kinds_gemm_graph_replay(L, m, k):
    """A grouped call whose weights have several kinds (the two row sets of
    channel-mixed linears) launches one GEMM per kind on the caller's stream
    (at k = 8192 each splits K and adds a reduce launch).  Captured into a HIP
    graph after an eager call, every replay -- with eager work and cleared
    outputs in between -- reproduces the eager outputs bit for bit."""
    specs = GROUP_SETS["channel_mix"]
    ns = [300, 64, 520, 130]
    X = SI.bf16_normal(9500 + m, (m, k))
    qws = [_quant_pair(L, SI.gaussian_weights(9510 + i, n, k, outlier_seed=9520 + i), *spec)[0]
           for i, (spec, n) in enumerate(zip(specs, ns))]
    Xd = to_dev_bf16(X)
    outs = [torch.empty((m, n), dtype=torch.bfloat16, device=DEV) for n in ns]
    L.lbq_linear_fwd_grouped(Xd, qws, outs=outs)
    torch.cuda.synchronize()
    ref = [bf16_bits_host(y) for y in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        L.lbq_linear_fwd_grouped(Xd, qws, outs=outs)
    for rep in range(4):
        for y in outs:
            y.zero_()
        junk = torch.randn(1 << 20, device=DEV).sum()  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert float(junk) == float(junk)
        for i, y in enumerate(outs):
            assert np.array_equal(bf16_bits_host(y), ref[i]), f"replay {rep} weight {i}"


@pytest.mark.parametrize("fid", ["i4g128", "nf4dq", "i2g64"])
def test_grouped_gemm_two_launch_split(L, fid):
    """A q/k/v-like set at ragged m = 4000 whose GEMM runs as two launches:
    the 4000-row weight alone fills one round of 256x256 tiles (256 tiles),
    the two 1000-row weights one round of 256x128 tiles.  Each output equals
    the single-weight forward bit for bit, and 48 sampled rows match the
    oracle."""
    fmt, bits, group, dq = FORMATS[FMT_IDS.index(fid)]
    m, k = 4000, 256
    rows = np.sort(np.random.default_rng(9460).choice(m, 48, replace=False))
    X = SI.bf16_normal(9461, (m, k))
    qws, refs = [], []
    for i, n in enumerate((4000, 1000, 1000)):
        qw, ref = _quant_pair(L, SI.gaussian_weights(9462 + i, n, k, outlier_seed=9465 + i), fmt, bits, group, dq)
        qws.append(qw)
        refs.append(ref)
    Xd = to_dev_bf16(X)
    Ys = L.lbq_linear_fwd_grouped(Xd, qws)
    singles = [L.lbq_linear_fwd(Xd, q) for q in qws]
    torch.cuda.synchronize()
    for i, (Y, Y1, ref) in enumerate(zip(Ys, singles, refs)):
        assert np.array_equal(bf16_bits_host(Y), bf16_bits_host(Y1)), f"{fid} weight {i}: grouped != single"
        assert_close(bf16_bits_host(Y)[rows], O.linear_fwd(X[rows], ref["w_exact"]), what=f"{fid} weight {i}")


@pytest.mark.parametrize("fid", FMT_IDS)
def test_grouped_gemm_row_cut(L, fid):
    """Two 2560-row weights at ragged m = 4000 have 320 tiles of 256x256 (one
    round and a quarter), so the set runs as two launches cut inside the
    second weight at row 1536: the first launch fills one round of 256x256
    tiles, the second (its last 1024 rows) takes its own tile shape.  Each
    output equals the single-weight forward bit for bit, and 48 sampled rows
    match the oracle.  With out_rows on the cut weight, its rows scatter into
    a wider Y exactly as the single-weight call scatters them."""
    fmt, bits, group, dq = FORMATS[FMT_IDS.index(fid)]
    m, k, n = 4000, 256, 2560
    rows = np.sort(np.random.default_rng(9470).choice(m, 48, replace=False))
    X = SI.bf16_normal(9471, (m, k))
    qws, refs = [], []
    for i in range(2):
        qw, ref = _quant_pair(L, SI.gaussian_weights(9472 + i, n, k, outlier_seed=9474 + i), fmt, bits, group, dq)
        qws.append(qw)
        refs.append(ref)
    Xd = to_dev_bf16(X)
    Ys = L.lbq_linear_fwd_grouped(Xd, qws)
    singles = [L.lbq_linear_fwd(Xd, q) for q in qws]
    torch.cuda.synchronize()
    for i, (Y, Y1, ref) in enumerate(zip(Ys, singles, refs)):
        assert np.array_equal(bf16_bits_host(Y), bf16_bits_host(Y1)), f"{fid} weight {i}: grouped != single"
        assert_close(bf16_bits_host(Y)[rows], O.linear_fwd(X[rows], ref["w_exact"]), what=f"{fid} weight {i}")
    cols = np.random.default_rng(9476).permutation(n + 64)[:n].astype(np.int32)
    qws[1].out_rows = torch.from_numpy(cols).to(DEV)
    Yg = torch.zeros((m, n + 64), dtype=torch.bfloat16, device=DEV)
    Y1 = torch.zeros((m, n + 64), dtype=torch.bfloat16, device=DEV)
    L.lbq_linear_fwd_grouped(Xd, qws, outs=[None, Yg])
    L.lbq_linear_fwd(Xd, qws[1], out=Y1)
    torch.cuda.synchronize()
    yg = bf16_bits_host(Yg)
    assert np.array_equal(yg, bf16_bits_host(Y1)), f"{fid}: scattered grouped != single"
    assert np.array_equal(yg[:, cols], bf16_bits_host(Ys[1])), f"{fid}: scattered columns"
    assert not np.any(np.delete(yg, cols, axis=1)), f"{fid}: columns outside out_rows written"


@pytest.mark.parametrize("fid", ["i4g64", "i4g128", "i2g64", "nf4", "nf4dq"])
def test_metadata_at_minimum_alignment(L, fid):
    """Metadata arrays that start one element past an aligned address (floats
    4-byte aligned, zero points and absmax codes 1-byte aligned, the least
    the API allows): the forward GEMM then loads one group's entries per stage
    instead of four groups' together.  Forward at m = 1, 16 and 300 and the
    input gradient equal those of the aligned weight bit for bit."""
    import dataclasses
    fmt, bits, group, dq = FORMATS[FMT_IDS.index(fid)]
    n, k = 520, 2048
    qw, _ = _quant_pair(L, SI.gaussian_weights(9480, n, k, outlier_seed=9481), fmt, bits, group, dq)

    def shifted(t):
        if t is None:
            return None
        buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)
        buf[1:].copy_(t.reshape(-1))
        return buf[1:].view(t.shape)

    qs = dataclasses.replace(qw, scales=shifted(qw.scales), zeros=shifted(qw.zeros),
                             absmax=shifted(qw.absmax), absmax_q=shifted(qw.absmax_q))
    for m in (1, 16, 300):
        X = to_dev_bf16(SI.bf16_normal(9482 + m, (m, k)))
        Y0, Y1 = L.lbq_linear_fwd(X, qw), L.lbq_linear_fwd(X, qs)
        torch.cuda.synchronize()
        assert np.array_equal(bf16_bits_host(Y0), bf16_bits_host(Y1)), f"{fid} fwd m={m}"
    dY = to_dev_bf16(SI.bf16_normal(9483, (300, n)))
    dX0, dX1 = L.lbq_linear_bwd_dx(dY, qw), L.lbq_linear_bwd_dx(dY, qs)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits_host(dX0), bf16_bits_host(dX1)), f"{fid} bwd"


def test_grouped_fwd_exact_on_grid(L):
    """Three grid weights in one m = 1 launch: exact integer arithmetic, so
    every output is bf16(X W_i^T) bit for bit."""
    k = 2048
    X = SI.bf16_small_ints(9450, (1, k))
    Ws = [SI.grid_weights(9451 + i, n, k, 128, 4) for i, n in enumerate((136, 8, 72))]
    qws = [_quant_pair(L, W, "minmax", 4, 128, False)[0] for W in Ws]
    Ys = L.lbq_linear_fwd_grouped(to_dev_bf16(X), qws)
    torch.cuda.synchronize()
    for W, Y in zip(Ws, Ys):
        exact = O.bf16_to_f64(X) @ W.astype(np.float64).T
        assert np.array_equal(bf16_bits_host(Y), O.bf16_bits(exact.astype(np.float32)))


# ------------------------------------------------------------------ serialization


@pytest.mark.parametrize("fmtspec", FORMATS, ids=FMT_IDS)
def test_serialize_round_trip(L, fmtspec):
    """Weight -> blob -> new device buffers: every stored byte, the dequantized
    weight and a forward are identical, and the blob's sections are the
    buffers' bytes at the offsets lbq.h documents."""
    fmt, bits, group, dq = fmtspec
    W = SI.gaussian_weights(9500, 37, 1280, outlier_seed=9501)
    qw, ref = _quant_pair(L, W, fmt, bits, group, dq)
    blob = qw.to_bytes()
    back = L.QuantizedWeight.from_bytes(blob, DEV)
    torch.cuda.synchronize()
    check_quantized_equal(back, ref, fmt, dq)
    assert bytes(back.desc) == bytes(qw.desc)
    # section offsets: header 96 bytes, then each buffer on a 16-byte boundary
    off = 96
    for t in (qw.packed, qw.scales, qw.zeros, qw.absmax, qw.absmax_q, qw.absmax_scale):
        if t is None:
            continue
        b = host(t).tobytes()
        assert blob[off:off + len(b)] == b
        off += (len(b) + 15) // 16 * 16
    assert off == len(blob)
    assert torch.equal(L.lbq_dequant(back).view(torch.int16), L.lbq_dequant(qw).view(torch.int16))
    X = to_dev_bf16(SI.bf16_normal(9502, (3, 1280)))
    assert torch.equal(L.lbq_linear_fwd(X, back).view(torch.int16), L.lbq_linear_fwd(X, qw).view(torch.int16))


@pytest.mark.parametrize("fmtspec", [FORMATS[0], FORMATS[1], FORMATS[5]], ids=["i4g128", "i2g64", "nf4dq"])
def test_packed_bytes_survive_a_bf16_storage(L, fmtspec):
    """The packed bytes held as bf16 (the float storage a sharding framework
    needs) and viewed back as bytes dequantize identically."""
    fmt, bits, group, dq = fmtspec
    W = SI.gaussian_weights(9510, 64, 1024)
    qw, _ = _quant_pair(L, W, fmt, bits, group, dq)
    as_bf16 = qw.storage_view(torch.bfloat16).clone()   # a separate float tensor
    assert as_bf16.dtype == torch.bfloat16 and as_bf16.numel() * 2 == qw.packed.numel()
    moved = L.QuantizedWeight(qw.desc, as_bf16.view(torch.uint8), qw.scales, qw.zeros, qw.absmax, qw.absmax_q,
                              qw.absmax_scale)
    assert torch.equal(L.lbq_dequant(moved).view(torch.int16), L.lbq_dequant(qw).view(torch.int16))


# ------------------------------------------------------------------ exact ties
# The rounding rules on inputs built to sit exactly on them (tests/tie_inputs.py):
# half-integer code, zero-point and double-quant quotients (round half to
# even) and NF4 values on a midpoint (the lower code).  The HIP quantizer must
# match the oracle and the exact-arithmetic expectation bit for bit.
import tie_inputs as TI


@pytest.mark.parametrize("bits,group", [(4, 128), (2, 64), (4, 64), (2, 128)],
                         ids=["i4g128", "i2g64", "i4g64", "i2g128"])
def test_quantize_minmax_ties_bitexact(L, bits, group):
    W, want = TI.minmax_tie_groups(bits, group)
    W = np.tile(W, (1, 2))  # two groups per row: the ties sit in both
    qw, ref = _quant_pair(L, W, "minmax", bits, group, False)
    wb = L.lbq_dequant(qw)
    torch.cuda.synchronize()
    check_quantized_equal(qw, ref, "minmax")
    assert np.array_equal(ref["codes"], np.tile(want["codes"], (1, 2)))
    assert np.array_equal(ref["zeros"], np.tile(want["zeros"], (1, 2)))
    assert np.array_equal(bf16_bits_host(wb), ref["w_bf16"])


def test_quantize_double_quant_ties_bitexact(L):
    """Blocks whose absmax values make every a / c2 an exact half-integer (or
    an integer): the int8 codes take the even neighbour."""
    a, want = TI.dq_tie_absmax(nblocks=512)
    W = np.zeros((512, 64), dtype=np.float32)
    W[np.arange(512), np.arange(512) % 64] = a                  # the block's absmax
    W[np.arange(512), (np.arange(512) + 7) % 64] = -a * np.float32(0.5)
    W = W.reshape(128, 256)
    qw, ref = _quant_pair(L, W, "nf4", 4, 64, True)
    wb = L.lbq_dequant(qw)
    torch.cuda.synchronize()
    check_quantized_equal(qw, ref, "nf4", True)
    assert np.array_equal(ref["absmax_q"], want["absmax_q"])
    assert np.array_equal(bf16_bits_host(wb), ref["w_bf16"])


@pytest.mark.parametrize("dq", [False, True], ids=["nf4", "nf4dq"])
def test_nf4_power_of_two_blocks_dequant_exact(L, dq):
    """Entries in {-a, 0, a}, a different per block and lossless under double
    quantization: the dequantized weight is W itself, bit for bit."""
    W = TI.nf4_power_of_two_blocks()
    qw, ref = _quant_pair(L, W, "nf4", 4, 64, dq)
    wb = L.lbq_dequant(qw)
    torch.cuda.synchronize()
    check_quantized_equal(qw, ref, "nf4", dq)
    assert np.array_equal(bf16_bits_host(wb), SI.to_bf16_bits(W))


@pytest.mark.parametrize("fmtspec", FORMATS, ids=FMT_IDS)
def test_quantize_subnormal_scales_bitexact(L, fmtspec):
    """Groups whose fp32 scale (or absmax, or second-level scale) is
    subnormal: the kernels keep denormals, so codes, metadata and the
    dequantized weight equal the oracle's bit for bit."""
    fmt, bits, group, dq = fmtspec
    rng = np.random.default_rng(4242)
    # rows 0..31 are one double-quant run of 256 blocks (its c2 is subnormal)
    W = (rng.uniform(-1.0, 1.0, size=(48, 512)) * np.float32(1e-38)).astype(np.float32)
    W[16:32] *= np.float32(1e-3)            # deep subnormals
    W[32:] = SI.gaussian_weights(4243, 16, 512)  # normal rows beside them
    W[40, :64] = np.float32(1e-45)           # the smallest subnormal
    qw, ref = _quant_pair(L, W, fmt, bits, group, dq)
    wb = L.lbq_dequant(qw)
    torch.cuda.synchronize()
    if fmt == "minmax":
        assert (ref["scales"] < np.float32(1.1754944e-38)).any()
    elif dq:
        assert ref["absmax_scale"][0] < np.float32(1.1754944e-38)
    check_quantized_equal(qw, ref, fmt, dq)
    assert np.array_equal(bf16_bits_host(wb), ref["w_bf16"])
