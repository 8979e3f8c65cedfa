"""GPU parity of the format variants against the oracle, through the C ABI:

* compact MinMax metadata (INT4 g128 and INT2 g64 with an fp16 scale rounded
  up and the zero points packed like the codes);
* NF4 with double quantization with a per-tensor offset.

Stored bytes and the dequantized weight are bit-exact; the forward (every
kernel: m = 1 GEMV, 2..4 multi-row GEMV, small batch, GEMM), the input
gradient, grouped calls and LoRA meet the matmul tolerance of the fp64
oracle, and on lossless grid inputs the matmuls are exact.
"""
import numpy as np
import pytest
import torch

import synth_inputs as SI
import tie_inputs as TI
from gpu_util import DEV, assert_close, bf16_bits_host, host, to_dev_bf16, to_dev_f32
from oracle import lbq_oracle as O

pytestmark = pytest.mark.gpu

VARIANTS = ["i4g128c", "i2g64c", "nf4dqo"]


@pytest.fixture(scope="module")
def L():
    import group_wise_minmax_amd as L
    assert torch.cuda.is_available()
    return L


def quant(L, W, variant):
    Wd = to_dev_f32(W)
    if variant == "i4g128c":
        return L.lbq_quantize(Wd, "minmax", 4, 128, compact=True)
    if variant == "i2g64c":
        return L.lbq_quantize(Wd, "minmax", 2, 64, compact=True)
    return L.lbq_quantize(Wd, "nf4", double_quant=True, dq_offset=True)


def check_stored(qw, ref, variant):
    assert np.array_equal(host(qw.packed), ref["packed"]), "packed bytes differ"
    if variant == "nf4dqo":
        assert np.array_equal(host(qw.absmax_q), ref["absmax_q"]), "absmax_q differ"
        assert np.array_equal(host(qw.absmax_scale).view(np.uint32), ref["absmax_scale"].view(np.uint32)), \
            "absmax_scale (with the offset) differ"
    else:
        s = host(qw.scales).view(np.uint16).reshape(ref["scales"].shape)
        assert np.array_equal(s, ref["scales"].view(np.uint16)), "fp16 scales differ"
        assert np.array_equal(host(qw.zeros).reshape(ref["zeros_packed"].shape), ref["zeros_packed"]), \
            "packed zero points differ"


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("shape", [(256, 256), (3, 512), (37, 1280), (1000, 4096), (130, 768)])
def test_variant_quantize_dequant_bitexact(L, variant, shape):
    n, k = shape
    W = SI.gaussian_weights(8000 + n, n, k, outlier_seed=8001 + n)
    qw = quant(L, W, variant)
    wb = L.lbq_dequant(qw)
    torch.cuda.synchronize()
    ref = O.quantize_variant(W, variant)
    check_stored(qw, ref, variant)
    assert np.array_equal(bf16_bits_host(wb), ref["w_bf16"])


@pytest.mark.parametrize("variant", VARIANTS)
def test_variant_special_values_bitexact(L, variant):
    """Heavy tails, all-zero rows, single-signed groups, tiny and subnormal
    ranges (fp16 subnormal scales, subnormal absmax data)."""
    rng = np.random.default_rng(8100)
    W = SI.student_t_weights(8101, 64, 1024)
    W[0] = 0.0
    W[1, :128] = -0.25
    W[2] = (rng.uniform(-1, 1, 1024) * 1e-6).astype(np.float32)   # fp16-subnormal scales
    W[3] = (rng.uniform(-1, 1, 1024) * 1e-38).astype(np.float32)  # fp32-subnormal values
    W[4, :64] = np.float32(1e-45)
    W[5] = (rng.uniform(-1, 1, 1024) * 3e5).astype(np.float32)    # scales past fp16 range saturate
    qw = quant(L, W, variant)
    wb = L.lbq_dequant(qw)
    torch.cuda.synchronize()
    ref = O.quantize_variant(W, variant)
    check_stored(qw, ref, variant)
    assert np.array_equal(bf16_bits_host(wb), ref["w_bf16"])


@pytest.mark.parametrize("variant", ["i4g128c", "i2g64c"])
def test_compact_ties_bitexact(L, variant):
    bits, group = (4, 128) if variant == "i4g128c" else (2, 64)
    W, want = TI.minmax_tie_groups(bits, group)
    W = np.tile(W, (1, 4))
    qw = quant(L, W, variant)
    torch.cuda.synchronize()
    ref = O.quantize_variant(W, variant)
    check_stored(qw, ref, variant)
    assert np.array_equal(ref["codes"], np.tile(want["codes"], (1, 4)))


def test_nf4dqo_offset_tree_and_ties_bitexact(L):
    """Absmax values whose offset-quantized codes are exact ties (the mean
    is exactly 0.5), and a tensor long enough that the offset's tree sum runs
    over many runs of 256 in the one-workgroup pass (nr = 4100 run sums)."""
    a, want = TI.offset_tie_absmax()
    W = np.zeros((a.size, 64), dtype=np.float32)
    W[np.arange(a.size), np.arange(a.size) % 64] = a
    W = W.reshape(-1, 256)
    qw = quant(L, W, "nf4dqo")
    torch.cuda.synchronize()
    ref = O.quantize_variant(W, "nf4dqo")
    check_stored(qw, ref, "nf4dqo")
    assert np.array_equal(ref["absmax_q"], want)
    W2 = SI.gaussian_weights(8200, 4100, 1024, outlier_seed=8201)  # 65600 blocks -> 257 runs
    W2 = np.concatenate([W2] * 16)                                 # 1049600 blocks -> 4100 runs
    qw2 = quant(L, W2, "nf4dqo")
    torch.cuda.synchronize()
    nb = W2.size // 64
    a2 = np.abs(W2.reshape(-1, 64)).max(1).astype(np.float32)
    off = O.absmax_offset(a2)
    got = host(qw2.absmax_scale)
    assert got.shape == (-(-nb // 256) + 1,)
    assert got[-1].view(np.uint32) == np.float32(off).view(np.uint32)
    q2, c2, _ = O.double_quant_offset(a2, 256)
    assert np.array_equal(host(qw2.absmax_q), q2)
    assert np.array_equal(got[:-1].view(np.uint32), c2.view(np.uint32))


FWD_M = [1, 2, 3, 4, 5, 16, 33, 64, 65, 130]


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("nk", [(300, 512), (1040, 1280)])
@pytest.mark.parametrize("m", FWD_M)
def test_variant_forward_tolerance(L, variant, nk, m):
    n, k = nk
    W = SI.gaussian_weights(8300 + n, n, k, outlier_seed=8301 + n)
    X = SI.bf16_normal(8302 + m, (m, k))
    qw = quant(L, W, variant)
    Y = L.lbq_linear_fwd(to_dev_bf16(X), qw)
    torch.cuda.synchronize()
    ref = O.quantize_variant(W, variant)
    assert_close(bf16_bits_host(Y), O.linear_fwd(X, ref["w_exact"]), what=f"{variant} n={n} k={k} m={m}")
    if 2 <= m <= 64:
        Yn = L.lbq_linear_fwd_noalloc(to_dev_bf16(X), qw)
        torch.cuda.synchronize()
        assert np.array_equal(bf16_bits_host(Yn), bf16_bits_host(Y))


@pytest.mark.parametrize("variant", ["i4g128c", "i2g64c"])
@pytest.mark.parametrize("m", [1, 3, 16, 130])
def test_compact_grid_matmuls_exact(L, variant, m):
    """Lossless grid weights (scale 2^-4, exact in fp16) and small-integer X:
    every partial sum is exact in fp32, so Y and dX equal bf16(exact)."""
    bits, group = (4, 128) if variant == "i4g128c" else (2, 64)
    W = SI.grid_weights(8400, 192, 512, group, bits)
    X = SI.bf16_small_ints(8401 + m, (m, 512))
    dY = SI.bf16_small_ints(8402 + m, (m, 192))
    qw = quant(L, W, variant)
    Y = L.lbq_linear_fwd(to_dev_bf16(X), qw)
    dX = L.lbq_linear_bwd_dx(to_dev_bf16(dY), qw)
    torch.cuda.synchronize()
    Wf = W.astype(np.float64)
    assert np.array_equal(bf16_bits_host(Y), O.bf16_bits((O.bf16_to_f64(X) @ Wf.T).astype(np.float32)))
    assert np.array_equal(bf16_bits_host(dX), O.bf16_bits((O.bf16_to_f64(dY) @ Wf).astype(np.float32)))


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("m", [3, 130])
def test_variant_bwd_tolerance(L, variant, m):
    n, k = 512, 1280
    W = SI.gaussian_weights(8500, n, k, outlier_seed=8501)
    dY = SI.bf16_normal(8502 + m, (m, n))
    qw = quant(L, W, variant)
    dX = L.lbq_linear_bwd_dx(to_dev_bf16(dY), qw)
    torch.cuda.synchronize()
    ref = O.quantize_variant(W, variant)
    assert_close(bf16_bits_host(dX), O.linear_bwd_dx(dY, ref["w_exact"]), what=f"{variant} bwd m={m}")


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("m", [1, 3, 16, 130])
def test_variant_grouped_equals_single(L, variant, m):
    """Three weights of one variant that share X: each grouped output equals
    the single-weight call bit for bit; the summed input gradient is within
    tolerance of the oracle."""
    k = 1024
    qws, refs = [], []
    for i, n in enumerate((512, 256, 320)):
        W = SI.gaussian_weights(8600 + i, n, k, outlier_seed=8610 + i)
        qws.append(quant(L, W, variant))
        refs.append(O.quantize_variant(W, variant))
    X = to_dev_bf16(SI.bf16_normal(8620 + m, (m, k)))
    Ys = L.lbq_linear_fwd_grouped(X, qws)
    for q, Yg in zip(qws, Ys):
        Y1 = L.lbq_linear_fwd(X, q)
        assert torch.equal(Yg.view(torch.int16), Y1.view(torch.int16))
    dYs = [SI.bf16_normal(8630 + i, (m, q.n)) for i, q in enumerate(qws)]
    dX = L.lbq_linear_bwd_dx_grouped([to_dev_bf16(d) for d in dYs], qws)
    torch.cuda.synchronize()
    assert_close(bf16_bits_host(dX), O.linear_bwd_dx_grouped(dYs, [r["w_exact"] for r in refs]),
                 what=f"{variant} grouped bwd m={m}")


@pytest.mark.parametrize("variant", VARIANTS)
def test_variant_grouped_row_cut(L, variant):
    """Two 2560-row weights at m = 4000: 320 tiles of 256x256, so a set of a
    compact kind runs as two launches cut inside the second weight at row
    1536 (the fp16 scales and packed zero points read from that row on).  The
    offset kind is never cut (its offset entry is found from the weight's row
    count).  Either way each grouped output equals the single-weight call bit
    for bit, and 32 sampled rows match the oracle."""
    m, k, n = 4000, 256, 2560
    rows = np.sort(np.random.default_rng(8680).choice(m, 32, replace=False))
    Xh = SI.bf16_normal(8681, (m, k))
    qws, refs = [], []
    for i in range(2):
        W = SI.gaussian_weights(8682 + i, n, k, outlier_seed=8684 + i)
        qws.append(quant(L, W, variant))
        refs.append(O.quantize_variant(W, variant))
    X = to_dev_bf16(Xh)
    Ys = L.lbq_linear_fwd_grouped(X, qws)
    singles = [L.lbq_linear_fwd(X, q) for q in qws]
    torch.cuda.synchronize()
    for i, (Yg, Y1, ref) in enumerate(zip(Ys, singles, refs)):
        assert torch.equal(Yg.view(torch.int16), Y1.view(torch.int16)), f"{variant} weight {i}"
        assert_close(bf16_bits_host(Yg)[rows], O.linear_fwd(Xh[rows], ref["w_exact"]), what=f"{variant} weight {i}")


@pytest.mark.parametrize("m", [1, 16, 130])
def test_nf4dqo_lora_fwd_bwd(L, m):
    n, k, r = 512, 1024, 16
    W = SI.gaussian_weights(8700, n, k, outlier_seed=8701)
    X = SI.bf16_normal(8702 + m, (m, k))
    dY = SI.bf16_normal(8703 + m, (m, n))
    A = SI.bf16_normal(8704, (r, k), std=0.01)
    B = SI.bf16_normal(8705, (n, r), std=0.01)
    qw = quant(L, W, "nf4dqo")
    ref = O.quantize_variant(W, "nf4dqo")
    Y = L.lbq_lora_fwd(to_dev_bf16(X), qw, to_dev_bf16(A), to_dev_bf16(B), 1.0)
    dX, dA, dB = L.lbq_lora_bwd(to_dev_bf16(X), to_dev_bf16(dY), qw, to_dev_bf16(A), to_dev_bf16(B), 1.0)
    torch.cuda.synchronize()
    assert_close(bf16_bits_host(Y), O.lora_fwd(X, ref["w_exact"], A, B, 1.0), what=f"nf4dqo lora m={m}")
    rX, rA, rB = O.lora_bwd(X, dY, ref["w_exact"], A, B, 1.0)
    assert_close(bf16_bits_host(dX), rX, what=f"nf4dqo lora bwd dX m={m}")
    for got, want in ((dA, rA), (dB, rB)):
        fro, mx = O.rel_errors(host(got).astype(np.float64), want)
        assert fro <= 5e-3 and mx <= 2e-2


@pytest.mark.parametrize("variant", VARIANTS)
def test_variant_serialization_roundtrip(L, variant):
    W = SI.gaussian_weights(8800, 96, 1024)
    qw = quant(L, W, variant)
    blob = qw.to_bytes()
    back = L.QuantizedWeight.from_bytes(blob, DEV)
    torch.cuda.synchronize()
    for a, b in ((qw.packed, back.packed), (qw.scales, back.scales), (qw.zeros, back.zeros),
                 (qw.absmax_q, back.absmax_q), (qw.absmax_scale, back.absmax_scale)):
        if a is not None:
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))
    assert torch.equal(L.lbq_dequant(qw).view(torch.int16), L.lbq_dequant(back).view(torch.int16))
