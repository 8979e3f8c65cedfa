"""Full-size parity: the LLaMA-3-8B, 70B-shaped and Qwen1.5-110B-shaped layers,
generated with the same seeds and launched through the same calls (hence the
same kernels and tile choices) as the benchmark, checked against the oracle.

Where the oracle can afford the whole weight (the 8B NF4 + double-quant
layer) every stored byte is compared; elsewhere rows of W are sampled (groups
and NF4 blocks never straddle rows, so a row's codes and metadata depend on
that row alone) together with rows of X, and the matmul outputs at the
sampled (row, column) pairs are checked to the fp64 tolerance.
"""
import numpy as np
import pytest
import torch

import group_wise_minmax_amd as L
import synth_inputs as SI
from gpu_util import DEV, assert_close, bf16_bits_host, host
from oracle import lbq_oracle as O

pytestmark = pytest.mark.gpu

NAMES = list(SI.LLAMA3_8B)


def sample(n: int, count: int, seed: int) -> np.ndarray:
    """`count` distinct indices in [0, n) plus the first and the last, sorted."""
    rng = np.random.default_rng(seed)
    idx = rng.choice(n, size=min(count, n), replace=False)
    return np.unique(np.concatenate([idx, [0, n - 1]])).astype(np.int64)


def rows_host(t: torch.Tensor, rows: np.ndarray) -> np.ndarray:
    return t[torch.from_numpy(rows).to(t.device)].cpu().numpy()


def bf16_rows(t: torch.Tensor, rows: np.ndarray) -> np.ndarray:
    return bf16_bits_host(t[torch.from_numpy(rows).to(t.device)])


def check_minmax_rows(qw, ref: dict, rows: np.ndarray, what: str):
    """Codes and metadata of the sampled rows, bit for bit."""
    r = torch.from_numpy(rows).to(DEV)
    assert np.array_equal(host(qw.packed[r]), ref["packed"]), f"{what}: packed bytes differ"
    s = host(qw.scales[r]).reshape(ref["scales"].shape)
    assert np.array_equal(s.view(np.uint32), ref["scales"].view(np.uint32)), f"{what}: scales differ"
    assert np.array_equal(host(qw.zeros[r]).reshape(ref["zeros"].shape), ref["zeros"]), f"{what}: zeros differ"


# ---------------------------------------------------------------------------
# LLaMA-3-8B layer, INT4 MinMax g128: quantize, dequant, GEMV m=1/16, GEMM m=2048
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("li", range(7), ids=NAMES)
def test_8b_int4_layer(li):
    nm = NAMES[li]
    n, k = SI.LLAMA3_8B[nm]
    W = SI.dev_gaussian_weights(SI.seed_of(2, li, SI.SLOT_W), n, k, DEV)
    qw = L.QuantizedWeight.empty(L.make_desc("minmax", n, k, 4, 128), DEV)
    L.lbq_quantize(W, "minmax", 4, 128, out=qw)
    rows = sample(n, 96, 7000 + li)
    ref = O.quantize(rows_host(W, rows), "minmax", bits=4, group=128)
    check_minmax_rows(qw, ref, rows, f"{nm} int4")

    wbf = torch.empty((n, k), dtype=torch.bfloat16, device=DEV)
    L.lbq_dequant(qw, out=wbf)
    assert np.array_equal(bf16_rows(wbf, rows), ref["w_bf16"]), f"{nm}: dequant differs"
    del wbf, W

    w_ref = ref["w_exact"]
    cols = torch.from_numpy(rows).to(DEV)
    for m, seed_off in ((1, 0), (16, 100), (2048, 200)):
        X = SI.dev_bf16_normal(SI.seed_of(2, li, SI.SLOT_X) + seed_off, (m, k), DEV)
        Y = L.lbq_linear_fwd(X, qw)
        torch.cuda.synchronize()
        ms = np.arange(m) if m <= 16 else sample(m, 64, 7100 + li)
        Xh = bf16_rows(X, ms)
        Yh = bf16_bits_host(Y[torch.from_numpy(ms).to(DEV)][:, cols])
        assert_close(Yh, O.linear_fwd(Xh, w_ref), what=f"{nm} int4 m={m}")


# ---------------------------------------------------------------------------
# LLaMA-3-8B layer, NF4 + double quant: every stored byte, dequant, forward
# m=4096, LoRA r=16 on q and v, input gradient m=4096
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("li", range(7), ids=NAMES)
def test_8b_nf4dq_layer(li):
    nm = NAMES[li]
    n, k = SI.LLAMA3_8B[nm]
    W = SI.dev_gaussian_weights(SI.seed_of(2, li, SI.SLOT_W), n, k, DEV)
    qw = L.QuantizedWeight.empty(L.make_desc("nf4", n, k, double_quant=True), DEV)
    L.lbq_quantize(W, "nf4", double_quant=True, out=qw)
    ref = O.quantize(W.cpu().numpy(), "nf4", double_quant_on=True)
    del W
    assert np.array_equal(host(qw.packed), ref["packed"]), f"{nm}: packed bytes differ"
    assert np.array_equal(host(qw.absmax_q), ref["absmax_q"]), f"{nm}: absmax_q differ"
    assert np.array_equal(host(qw.absmax_scale).view(np.uint32), ref["absmax_scale"].view(np.uint32)), \
        f"{nm}: absmax_scale differ"

    rows = sample(n, 128, 7200 + li)
    wbf = torch.empty((n, k), dtype=torch.bfloat16, device=DEV)
    L.lbq_dequant(qw, out=wbf)
    assert np.array_equal(bf16_rows(wbf, rows), ref["w_bf16"][rows]), f"{nm}: dequant differs"
    del wbf
    w_ref = ref["w_exact"]
    del ref

    m = 4096
    ms = sample(m, 64, 7300 + li)
    ms_t = torch.from_numpy(ms).to(DEV)
    X = SI.dev_bf16_normal(SI.seed_of(3, li, SI.SLOT_X), (m, k), DEV)
    Y = L.lbq_linear_fwd(X, qw)
    Xh = bf16_rows(X, ms)
    assert_close(bf16_bits_host(Y[ms_t]), O.linear_fwd(Xh, w_ref), what=f"{nm} nf4dq fwd m={m}")
    del Y

    if nm in ("q", "v"):
        A = SI.dev_bf16_normal(SI.seed_of(3, li, SI.SLOT_A), (16, k), DEV, std=0.01)
        B = SI.dev_bf16_normal(SI.seed_of(3, li, SI.SLOT_B), (n, 16), DEV, std=0.01)
        ws = torch.empty(L.lbq_lora_workspace_bytes(qw, m, 16), dtype=torch.uint8, device=DEV)
        Yl = L.lbq_lora_fwd(X, qw, A, B, 1.0, workspace=ws)
        ref_l = O.lora_fwd(Xh, w_ref, bf16_bits_host(A), bf16_bits_host(B), 1.0)
        assert_close(bf16_bits_host(Yl[ms_t]), ref_l, what=f"{nm} lora m={m}")
        del Yl
    dY = SI.dev_bf16_normal(SI.seed_of(3, li, SI.SLOT_DY), (m, n), DEV)
    if nm in ("q", "v"):
        # LoRA backward: dX on the sampled rows, dA and dB in full (they sum over all m rows).
        dXl, dA, dB = L.lbq_lora_bwd(X, dY, qw, A, B, 1.0)
        Ah, Bh = bf16_bits_host(A), bf16_bits_host(B)
        rX, _, _ = O.lora_bwd(Xh, bf16_rows(dY, ms), w_ref, Ah, Bh, 1.0)
        assert_close(bf16_bits_host(dXl[ms_t]), rX, what=f"{nm} lora bwd dX m={m}")
        del dXl
        _, rA, rB = O.lora_bwd(bf16_bits_host(X), bf16_bits_host(dY), np.zeros((n, k)), Ah, Bh, 1.0)
        for got, want, what in ((dA, rA, "dA"), (dB, rB, "dB")):
            fro, mx = O.rel_errors(host(got).astype(np.float64), want)
            assert fro <= 5e-3 and mx <= 2e-2, f"{nm} lora bwd {what}: rel_fro={fro:.3e} max_rel={mx:.3e}"
    del X

    dX = L.lbq_linear_bwd_dx(dY, qw)
    assert_close(bf16_bits_host(dX[ms_t]), O.linear_bwd_dx(bf16_rows(dY, ms), w_ref),
                 what=f"{nm} nf4dq bwd m={m}")


@pytest.mark.parametrize("group", [("q", "k", "v"), ("gate", "up")], ids=["qkv", "gate_up"])
def test_8b_grouped_bwd(group):
    """The layer's summed input gradients as the grouped backward phase runs
    them (NF4+DQ, m = 4096, one launch per group): 64 sampled rows of dX
    against the oracle's sum over the group's weights."""
    m = 4096
    ms = sample(m, 64, 7600 + len(group))
    ms_t = torch.from_numpy(ms).to(DEV)
    qws, w_refs, dYs = [], [], []
    for nm in group:
        li = NAMES.index(nm)
        n, k = SI.LLAMA3_8B[nm]
        W = SI.dev_gaussian_weights(SI.seed_of(2, li, SI.SLOT_W), n, k, DEV)
        qws.append(L.lbq_quantize(W, "nf4", double_quant=True))
        w_refs.append(O.quantize(W.cpu().numpy(), "nf4", double_quant_on=True)["w_exact"])
        del W
        dYs.append(SI.dev_bf16_normal(SI.seed_of(3, li, SI.SLOT_DY), (m, n), DEV))
    dX = L.lbq_linear_bwd_dx_grouped(dYs, qws)
    ref = O.linear_bwd_dx_grouped([bf16_rows(d, ms) for d in dYs], w_refs)
    assert_close(bf16_bits_host(dX[ms_t]), ref, what=f"{'+'.join(group)} grouped bwd m={m}")
    del dX, dYs, qws
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# LLaMA-3-8B layer, linears that share X in one launch (q/k/v, gate/up), as the
# benchmark runs them: bit-identical to one launch per linear (whose outputs
# the tests above check against the oracle)
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("fmt,m", [("int4", 1), ("nf4dq", 1), ("nf4dq", 4096), ("int4", 2048)])
def test_8b_grouped_matches_single(fmt, m):
    for group in (("q", "k", "v"), ("gate", "up")):
        qws = []
        for nm in group:
            li = NAMES.index(nm)
            n, k = SI.LLAMA3_8B[nm]
            W = SI.dev_gaussian_weights(SI.seed_of(2, li, SI.SLOT_W), n, k, DEV)
            if fmt == "int4":
                qws.append(L.lbq_quantize(W, "minmax", 4, 128))
            else:
                qws.append(L.lbq_quantize(W, "nf4", double_quant=True))
            del W
        k = qws[0].k
        X = SI.dev_bf16_normal(SI.seed_of(3, NAMES.index(group[0]), SI.SLOT_X), (m, k), DEV)
        Ys = L.lbq_linear_fwd_grouped(X, qws)
        for nm, q, Y in zip(group, qws, Ys):
            Y1 = L.lbq_linear_fwd(X, q)
            assert torch.equal(Y.view(torch.int16), Y1.view(torch.int16)), f"{fmt} {nm} m={m}: grouped != single"
        del Ys, qws, X
        torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# 70B-shaped layer, channel-mix 25% INT4 g128 / 75% INT2 g64, m = 1 and 1024
# ---------------------------------------------------------------------------

NAMES70 = list(SI.LLAMA3_70B)


@pytest.mark.parametrize("li", range(7), ids=NAMES70)
def test_70b_channel_mix_layer(li):
    nm = NAMES70[li]
    n, k = SI.LLAMA3_70B[nm]
    W = SI.dev_gaussian_weights(SI.seed_of(4, li, SI.SLOT_W), n, k, DEV)
    rows4 = SI.dev_channel_mask(SI.seed_of(4, li, SI.SLOT_CHMASK), n, DEV)
    mask = torch.zeros(n, dtype=torch.bool, device=DEV)
    mask[rows4.long()] = True
    rows2 = torch.nonzero(~mask).flatten().to(torch.int32)
    a = L.lbq_quantize(W[rows4.long()].contiguous(), "minmax", 4, 128)
    b = L.lbq_quantize(W[rows2.long()].contiguous(), "minmax", 2, 64)
    a.out_rows, b.out_rows = rows4, rows2

    # Sampled output columns, each quantized by the oracle in its own format.
    cols = sample(n, 128, 7400 + li)
    is4 = host(mask)[cols]
    Wc = rows_host(W, cols)
    del W
    w_ref = np.empty((len(cols), k), dtype=np.float64)
    if is4.any():
        w_ref[is4] = O.quantize(Wc[is4], "minmax", bits=4, group=128)["w_exact"]
    w_ref[~is4] = O.quantize(Wc[~is4], "minmax", bits=2, group=64)["w_exact"]
    cols_t = torch.from_numpy(cols).to(DEV)

    for m, seed_off in ((1, 0), (1024, 100)):
        X = SI.dev_bf16_normal(SI.seed_of(4, li, SI.SLOT_X) + seed_off, (m, k), DEV)
        Y = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
        L.lbq_linear_fwd(X, a, out=Y)
        L.lbq_linear_fwd(X, b, out=Y)
        ms = np.arange(m) if m == 1 else sample(m, 64, 7500 + li)
        Yh = bf16_bits_host(Y[torch.from_numpy(ms).to(DEV)][:, cols_t])
        assert_close(Yh, O.linear_fwd(bf16_rows(X, ms), w_ref), what=f"70b {nm} chmix m={m}")


@pytest.mark.parametrize("grp", [("q", "k", "v"), ("gate", "up"), ("down",)], ids=["qkv", "gate_up", "down"])
def test_70b_channel_mix_small_batch_one_launch(grp):
    """The channel-mixed linears that share X as the bench runs them at
    m = 3, 16 and 40: both formats of every linear in one grouped call (one
    small-batch launch plus its reduce) equal the per-format calls bit for
    bit, and sampled columns meet the oracle's tolerance."""
    parts, refs = [], []
    for nm in grp:
        li = NAMES70.index(nm)
        n, k = SI.LLAMA3_70B[nm]
        W = SI.dev_gaussian_weights(SI.seed_of(4, li, SI.SLOT_W), n, k, DEV)
        rows4 = SI.dev_channel_mask(SI.seed_of(4, li, SI.SLOT_CHMASK), n, DEV)
        mask = torch.zeros(n, dtype=torch.bool, device=DEV)
        mask[rows4.long()] = True
        rows2 = torch.nonzero(~mask).flatten().to(torch.int32)
        a = L.lbq_quantize(W[rows4.long()].contiguous(), "minmax", 4, 128)
        b = L.lbq_quantize(W[rows2.long()].contiguous(), "minmax", 2, 64)
        a.out_rows, b.out_rows = rows4, rows2
        cols = sample(n, 48, 8100 + li)
        is4 = host(mask)[cols]
        Wc = rows_host(W, cols)
        w_ref = np.empty((len(cols), k), dtype=np.float64)
        if is4.any():
            w_ref[is4] = O.quantize(Wc[is4], "minmax", bits=4, group=128)["w_exact"]
        w_ref[~is4] = O.quantize(Wc[~is4], "minmax", bits=2, group=64)["w_exact"]
        del W
        parts.append((nm, n, a, b))
        refs.append((cols, w_ref))
    k = parts[0][2].k
    for m in (3, 16, 40):
        X = SI.dev_bf16_normal(SI.seed_of(4, NAMES70.index(grp[0]), SI.SLOT_X) + 300 + m, (m, k), DEV)
        Yg = [torch.zeros((m, n), dtype=torch.bfloat16, device=DEV) for _, n, _, _ in parts]
        L.lbq_linear_fwd_grouped(X, [q for _, _, a, b in parts for q in (a, b)], outs=[y for y in Yg for _ in range(2)])
        Xh = bf16_bits_host(X)
        for (nm, n, a, b), y, (cols, w_ref) in zip(parts, Yg, refs):
            Ys = torch.zeros((m, n), dtype=torch.bfloat16, device=DEV)
            L.lbq_linear_fwd(X, a, out=Ys)
            L.lbq_linear_fwd(X, b, out=Ys)
            torch.cuda.synchronize()
            assert torch.equal(y.view(torch.int16), Ys.view(torch.int16)), f"70b {nm} m={m}: one launch != per format"
            Yh = bf16_bits_host(y[:, torch.from_numpy(cols).to(DEV)])
            assert_close(Yh, O.linear_fwd(Xh, w_ref), what=f"70b {nm} chmix m={m}")
    torch.cuda.empty_cache()


@pytest.mark.parametrize("grp", [("q", "k", "v"), ("o",), ("down",)], ids=["qkv", "o", "down"])
def test_8b_channel_mix_multirow_one_launch(grp):
    """Channel-mixed 8B-shaped linears (25% INT4 g128 / 75% INT2 g64 rows) that
    share X, at m = 2 and 4 where every row set takes the multi-row GEMV (down,
    k = 14336, only at m = 2): both formats of every linear in one grouped call
    -- one mixed multi-row launch -- equal the per-format calls bit for bit,
    and sampled columns meet the oracle's tolerance."""
    parts, refs = [], []
    for nm in grp:
        li = NAMES.index(nm)
        n, k = SI.LLAMA3_8B[nm]
        W = SI.dev_gaussian_weights(SI.seed_of(5, li, SI.SLOT_W), n, k, DEV)
        rows4 = SI.dev_channel_mask(SI.seed_of(5, li, SI.SLOT_CHMASK), n, DEV)
        mask = torch.zeros(n, dtype=torch.bool, device=DEV)
        mask[rows4.long()] = True
        rows2 = torch.nonzero(~mask).flatten().to(torch.int32)
        a = L.lbq_quantize(W[rows4.long()].contiguous(), "minmax", 4, 128)
        b = L.lbq_quantize(W[rows2.long()].contiguous(), "minmax", 2, 64)
        a.out_rows, b.out_rows = rows4, rows2
        cols = sample(n, 48, 8300 + li)
        is4 = host(mask)[cols]
        Wc = rows_host(W, cols)
        w_ref = np.empty((len(cols), k), dtype=np.float64)
        if is4.any():
            w_ref[is4] = O.quantize(Wc[is4], "minmax", bits=4, group=128)["w_exact"]
        w_ref[~is4] = O.quantize(Wc[~is4], "minmax", bits=2, group=64)["w_exact"]
        del W
        parts.append((nm, n, a, b))
        refs.append((cols, w_ref))
    k = parts[0][2].k
    for m in ((2,) if k > 8192 else (2, 4)):
        X = SI.dev_bf16_normal(SI.seed_of(5, NAMES.index(grp[0]), SI.SLOT_X) + 400 + m, (m, k), DEV)
        Yg = [torch.zeros((m, n), dtype=torch.bfloat16, device=DEV) for _, n, _, _ in parts]
        L.lbq_linear_fwd_grouped(X, [q for _, _, a, b in parts for q in (a, b)], outs=[y for y in Yg for _ in range(2)])
        Xh = bf16_bits_host(X)
        for (nm, n, a, b), y, (cols, w_ref) in zip(parts, Yg, refs):
            Ys = torch.zeros((m, n), dtype=torch.bfloat16, device=DEV)
            L.lbq_linear_fwd(X, a, out=Ys)
            L.lbq_linear_fwd(X, b, out=Ys)
            torch.cuda.synchronize()
            assert torch.equal(y.view(torch.int16), Ys.view(torch.int16)), f"8b {nm} m={m}: one launch != per format"
            Yh = bf16_bits_host(y[:, torch.from_numpy(cols).to(DEV)])
            assert_close(Yh, O.linear_fwd(Xh, w_ref), what=f"8b {nm} chmix m={m}")
    torch.cuda.empty_cache()


@pytest.mark.parametrize("bits,group", [(4, 128), (2, 64)], ids=["int4", "int2"])
@pytest.mark.parametrize("li", range(7), ids=NAMES70)
def test_70b_layer_mix_layer(li, bits, group):
    """Layer-mix: the whole 70B-shaped linear in one format (every linear all
    INT4 g128, or all INT2 g64), m = 1 and 1024, sampled rows of codes and
    metadata bit for bit and sampled outputs against the oracle."""
    nm = NAMES70[li]
    n, k = SI.LLAMA3_70B[nm]
    W = SI.dev_gaussian_weights(SI.seed_of(4, li, SI.SLOT_W), n, k, DEV)
    qw = L.lbq_quantize(W, "minmax", bits, group)
    rows = sample(n, 96, 7800 + li + bits)
    ref = O.quantize(rows_host(W, rows), "minmax", bits=bits, group=group)
    del W
    check_minmax_rows(qw, ref, rows, f"70b {nm} int{bits}")
    cols = torch.from_numpy(rows).to(DEV)
    for m, seed_off in ((1, 0), (1024, 100)):
        X = SI.dev_bf16_normal(SI.seed_of(4, li, SI.SLOT_X) + seed_off, (m, k), DEV)
        Y = L.lbq_linear_fwd(X, qw)
        ms = np.arange(m) if m == 1 else sample(m, 64, 7900 + li)
        Yh = bf16_bits_host(Y[torch.from_numpy(ms).to(DEV)][:, cols])
        assert_close(Yh, O.linear_fwd(bf16_rows(X, ms), ref["w_exact"]), what=f"70b {nm} int{bits} m={m}")
    del qw
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# Qwen1.5-110B-shaped layer, INT2 g64, heavy-tailed weights: quantize the whole
# layer, GEMV m=1, GEMM m=512
# ---------------------------------------------------------------------------

NAMESQ = list(SI.QWEN15_110B)


@pytest.mark.parametrize("li", range(7), ids=NAMESQ)
def test_qwen_int2_layer(li):
    nm = NAMESQ[li]
    n, k = SI.QWEN15_110B[nm]
    W = SI.dev_student_t_weights(SI.seed_of(5, li, SI.SLOT_W), n, k, DEV)
    qw = L.QuantizedWeight.empty(L.make_desc("minmax", n, k, 2, 64), DEV)
    L.lbq_quantize(W, "minmax", 2, 64, out=qw)
    rows = sample(n, 96, 7600 + li)
    ref = O.quantize(rows_host(W, rows), "minmax", bits=2, group=64)
    del W
    check_minmax_rows(qw, ref, rows, f"qwen {nm} int2")
    cols = torch.from_numpy(rows).to(DEV)
    for m, seed_off in ((1, 0), (512, 100)):
        X = SI.dev_bf16_normal(SI.seed_of(5, li, SI.SLOT_X) + seed_off, (m, k), DEV)
        Y = L.lbq_linear_fwd(X, qw)
        ms = np.arange(m) if m == 1 else sample(m, 64, 7700 + li)
        Yh = bf16_bits_host(Y[torch.from_numpy(ms).to(DEV)][:, cols])
        assert_close(Yh, O.linear_fwd(bf16_rows(X, ms), ref["w_exact"]), what=f"qwen {nm} int2 m={m}")
