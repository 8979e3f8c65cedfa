"""Host-side checks of the C ABI: the library loads without a GPU, exports every
symbol include/lbq.h declares, computes buffer sizes by the closed forms, and
rejects every malformed request before touching the device."""
import ctypes
import os
import re

import numpy as np
import pytest

from oracle import lbq_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    import group_wise_minmax_amd as L
    return L


def declared_symbols():
    src = open(os.path.join(ROOT, "include", "lbq.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(lbq_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol(L):
    lib = ctypes.CDLL(L.LIB_PATH)
    decl = declared_symbols()
    assert len(decl) >= 12
    for name in decl:
        assert hasattr(lib, name), name
    assert set(decl) == set(L.EXPORTED)
    assert "gfx950" in L.version()


def test_library_exports_only_declared_symbols(L):
    """Every C-linkage symbol the library defines is one include/lbq.h declares
    (runtime-internal names start with an underscore)."""
    import shutil
    import subprocess
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm is not installed")
    out = subprocess.run([nm, "-D", "--defined-only", L.LIB_PATH], capture_output=True, text=True, check=True).stdout
    names = {ln.split()[-1] for ln in out.splitlines() if ln.strip()}
    extra = sorted(n for n in names if not n.startswith("_") and n not in set(declared_symbols()))
    assert not extra, extra


def test_nf4_codebook_matches_oracle(L):
    """The library builds its table itself (bisection on erfc); the oracle
    uses a different quantile routine.  After fp32 rounding they must agree."""
    lib_tab = np.array(L.lbq_nf4_codebook(), dtype=np.float32)
    assert np.array_equal(lib_tab, O.nf4_codebook())


@pytest.mark.parametrize("fmt,bits,group,dq,n,k", [
    ("minmax", 4, 128, False, 4096, 4096), ("minmax", 2, 64, False, 1024, 8192),
    ("minmax", 4, 64, False, 3, 192), ("minmax", 2, 128, False, 5, 384),
    ("nf4", 4, 64, True, 14336, 4096), ("nf4", 4, 64, False, 7, 64), ("nf4", 4, 64, True, 3, 320),
])
def test_layout_closed_forms(L, fmt, bits, group, dq, n, k):
    s = L.lbq_layout(L.make_desc(fmt, n, k, bits, group, dq))
    assert s["packed"] == n * k * bits // 8
    if fmt == "minmax":
        assert s["scales"] == 4 * n * k // group and s["zeros"] == n * k // group
        assert s["absmax"] == s["absmax_q"] == s["absmax_scale"] == 0
    else:
        nb = n * k // 64
        if dq:
            assert s["absmax_q"] == nb and s["absmax_scale"] == 4 * (-(-nb // 256)) and s["absmax"] == 0
        else:
            assert s["absmax"] == 4 * nb and s["absmax_q"] == 0
        assert s["scales"] == s["zeros"] == 0


def test_layout_double_quant_saving(L):
    """Bits per parameter saved by double quantization, from the library's own
    byte counts: 0.373046875 on every 8B / 70B / 110B shape."""
    import synth_inputs as SI
    for shapes in (SI.LLAMA3_8B, SI.LLAMA3_70B, SI.QWEN15_110B):
        for n, k in shapes.values():
            a = L.lbq_layout(L.make_desc("nf4", n, k, double_quant=False))
            b = L.lbq_layout(L.make_desc("nf4", n, k, double_quant=True))
            saved = a["absmax"] - (b["absmax_q"] + b["absmax_scale"])
            assert 8.0 * saved / (n * k) == 0.373046875


def test_layout_format_variants(L):
    """Compact MinMax metadata (fp16 scales, zero points packed like the
    codes) and double quantization with an offset (one more fp32 after the
    per-run scales): byte counts and bits per parameter by the closed forms."""
    import synth_inputs as SI
    for shapes in (SI.LLAMA3_8B, SI.LLAMA3_70B, SI.QWEN15_110B):
        for n, k in shapes.values():
            for bits, group, bpp in ((4, 128, 4.15625), (2, 64, 2.28125)):
                s = L.lbq_layout(L.make_desc("minmax", n, k, bits, group, compact=True))
                assert s["scales"] == 2 * n * (k // group) and s["zeros"] == n * (k // group) * bits // 8
                assert 8.0 * (s["packed"] + s["scales"] + s["zeros"]) / (n * k) == bpp
            nb = n * k // 64
            s = L.lbq_layout(L.make_desc("nf4", n, k, double_quant=True, dq_offset=True))
            assert s["absmax_q"] == nb and s["absmax_scale"] == 4 * (-(-nb // 256) + 1) and s["absmax"] == 0
    d = L.make_desc("nf4", 64, 256, double_quant=True, dq_offset=True)
    assert d.double_quant == 2 and d.dq_block == 256
    for bad in (dict(double_quant=3), dict(meta=1)):
        e = L.make_desc("nf4", 64, 256)
        for k_, v in bad.items():
            setattr(e, k_, v)
        with pytest.raises(L.LbqError) as err:
            L.lbq_layout(e)
        assert err.value.name == "LBQ_E_FORMAT"


def _desc(L, **kw):
    d = L.make_desc("minmax", 64, 256, 4, 128)
    for k, v in kw.items():
        setattr(d, k, v)
    return d


@pytest.mark.parametrize("kw,code", [
    (dict(format=7), "LBQ_E_FORMAT"), (dict(bits=3), "LBQ_E_FORMAT"), (dict(bits=8), "LBQ_E_FORMAT"),
    (dict(group=32), "LBQ_E_FORMAT"), (dict(group=100), "LBQ_E_FORMAT"),
    (dict(double_quant=1), "LBQ_E_FORMAT"), (dict(meta=2), "LBQ_E_FORMAT"), (dict(meta=-1), "LBQ_E_FORMAT"),
    (dict(meta=1, group=64), "LBQ_E_FORMAT"), (dict(meta=1, k=128), "LBQ_E_SHAPE"),
    (dict(n=0), "LBQ_E_SHAPE"), (dict(k=0), "LBQ_E_SHAPE"), (dict(k=96), "LBQ_E_SHAPE"),
    (dict(k=192), "LBQ_E_SHAPE"), (dict(n=-5), "LBQ_E_SHAPE"),
])
def test_layout_rejects_bad_desc(L, kw, code):
    with pytest.raises(L.LbqError) as e:
        L.lbq_layout(_desc(L, **kw))
    assert e.value.name == code


def test_nf4_type_check(L):
    """Only the nf4 type exists among 4-bit float types (fp4 is not built):
    a wrong quant type is a format error, as the type check in the
    bitsandbytes guide's parameter table makes it."""
    d = L.make_desc("nf4", 64, 256)
    d.bits = 2
    with pytest.raises(L.LbqError) as e:
        L.lbq_layout(d)
    assert e.value.name == "LBQ_E_FORMAT"
    d = L.make_desc("nf4", 64, 256)
    d.group = 128
    with pytest.raises(L.LbqError):
        L.lbq_layout(d)
    d = L.make_desc("nf4", 64, 256, double_quant=True)
    d.dq_block = 128
    with pytest.raises(L.LbqError):
        L.lbq_layout(d)


# Error paths of the device entry points: every one must be caught on the host
# before any launch, so fake (never dereferenced) addresses are enough here.
FAKE = 0x7F0000000000  # 16-byte aligned, never touched


def _q(L, **kw):
    q = L.QTensor()
    q.packed = FAKE
    q.scales = FAKE + 0x1000
    q.zeros = FAKE + 0x2000
    q.absmax = FAKE + 0x3000
    q.absmax_q = FAKE + 0x4000
    q.absmax_scale = FAKE + 0x5000
    for k, v in kw.items():
        setattr(q, k, v)
    return q


def _status(L, rc):
    return L._lib.STATUS[rc]


def test_quantize_error_paths(L):
    lib = L.lib
    d = L.make_desc("minmax", 64, 256)
    B = ctypes.byref
    assert _status(L, lib.lbq_quantize(None, FAKE, B(_q(L)), None)) == "LBQ_E_NULL"
    assert _status(L, lib.lbq_quantize(B(d), None, B(_q(L)), None)) == "LBQ_E_NULL"
    assert _status(L, lib.lbq_quantize(B(d), FAKE, None, None)) == "LBQ_E_NULL"
    assert _status(L, lib.lbq_quantize(B(d), FAKE, B(_q(L, packed=None)), None)) == "LBQ_E_NULL"
    assert _status(L, lib.lbq_quantize(B(d), FAKE, B(_q(L, scales=None)), None)) == "LBQ_E_NULL"
    assert _status(L, lib.lbq_quantize(B(d), FAKE, B(_q(L, zeros=None)), None)) == "LBQ_E_NULL"
    assert _status(L, lib.lbq_quantize(B(d), FAKE + 4, B(_q(L)), None)) == "LBQ_E_ALIGN"
    assert _status(L, lib.lbq_quantize(B(d), FAKE, B(_q(L, packed=FAKE + 8)), None)) == "LBQ_E_ALIGN"
    assert _status(L, lib.lbq_quantize(B(d), FAKE, B(_q(L, scales=FAKE + 2)), None)) == "LBQ_E_ALIGN"
    assert "16-byte" in lib.lbq_last_error_detail().decode() or "4-byte" in lib.lbq_last_error_detail().decode()
    dn = L.make_desc("nf4", 64, 256, double_quant=True)
    assert _status(L, lib.lbq_quantize(B(dn), FAKE, B(_q(L, absmax_q=None)), None)) == "LBQ_E_NULL"
    assert _status(L, lib.lbq_quantize(B(dn), FAKE, B(_q(L, absmax_scale=None)), None)) == "LBQ_E_NULL"
    dn0 = L.make_desc("nf4", 64, 256, double_quant=False)
    assert _status(L, lib.lbq_quantize(B(dn0), FAKE, B(_q(L, absmax=None)), None)) == "LBQ_E_NULL"


def test_dequant_error_paths(L):
    lib = L.lib
    d = L.make_desc("minmax", 64, 256, 2, 64)
    B = ctypes.byref
    assert _status(L, lib.lbq_dequant(B(d), B(_q(L)), None, None)) == "LBQ_E_NULL"
    assert _status(L, lib.lbq_dequant(B(d), B(_q(L)), FAKE + 2, None)) == "LBQ_E_ALIGN"
    bad = L.make_desc("minmax", 64, 256, 4, 128)
    bad.bits = 1
    assert _status(L, lib.lbq_dequant(B(bad), B(_q(L)), FAKE, None)) == "LBQ_E_FORMAT"


def test_fwd_error_paths(L):
    lib = L.lib
    d = L.make_desc("minmax", 64, 256)
    B = ctypes.byref
    q = _q(L)
    assert _status(L, lib.lbq_linear_fwd(B(d), B(q), FAKE, -1, FAKE, 64, None, 0, None)) == "LBQ_E_SHAPE"
    assert _status(L, lib.lbq_linear_fwd(B(d), B(q), None, 4, FAKE, 64, None, 0, None)) == "LBQ_E_NULL"
    assert _status(L, lib.lbq_linear_fwd(B(d), B(q), FAKE, 4, None, 64, None, 0, None)) == "LBQ_E_NULL"
    assert _status(L, lib.lbq_linear_fwd(B(d), B(q), FAKE + 2, 4, FAKE, 64, None, 0, None)) == "LBQ_E_ALIGN"
    assert _status(L, lib.lbq_linear_fwd(B(d), B(q), FAKE, 4, FAKE + 1, 64, None, 0, None)) == "LBQ_E_ALIGN"
    assert _status(L, lib.lbq_linear_fwd(B(d), B(q), FAKE, 4, FAKE, 60, None, 0, None)) == "LBQ_E_SHAPE"
    # m == 0 is an empty batch: a no-op that touches nothing
    assert _status(L, lib.lbq_linear_fwd(B(d), B(q), None, 0, None, 64, None, 0, None)) == "LBQ_OK"


def test_bwd_error_paths(L):
    lib = L.lib
    B = ctypes.byref
    d = L.make_desc("minmax", 64, 256)
    assert _status(L, lib.lbq_linear_bwd_dx(B(d), B(_q(L, out_rows=FAKE)), FAKE, 4, FAKE, None)) == "LBQ_E_UNSUPPORTED"
    assert _status(L, lib.lbq_linear_bwd_dx(B(d), B(_q(L)), None, 4, FAKE, None)) == "LBQ_E_NULL"
    assert _status(L, lib.lbq_linear_bwd_dx(B(d), B(_q(L)), FAKE + 8, 4, FAKE, None)) == "LBQ_E_ALIGN"
    d2 = L.make_desc("minmax", 60, 256)
    assert _status(L, lib.lbq_linear_bwd_dx(B(d2), B(_q(L)), FAKE, 4, FAKE, None)) == "LBQ_E_SHAPE"
    assert _status(L, lib.lbq_linear_bwd_dx(B(d), B(_q(L)), None, 0, None, None)) == "LBQ_OK"


def test_lora_error_paths(L):
    lib = L.lib
    B = ctypes.byref
    d = L.make_desc("nf4", 64, 256, double_quant=True)
    q = _q(L)
    need = lib.lbq_lora_workspace_bytes(B(d), 8, 16)
    # bf16 T [m][32], then fp32 partial sums of at least one [m][16] slice
    assert need >= 8 * 32 * 2 + 8 * 16 * 4 and need % 16 == 0
    assert lib.lbq_lora_workspace_bytes(B(d), 8, 33) >= need + 8 * 32 * 2  # rank padded to 64
    assert lib.lbq_lora_workspace_bytes(B(d), 1, 16) >= 1 * 32 * 2 + 16 * 4
    assert lib.lbq_lora_workspace_bytes(B(d), 8, 65) == 0
    assert lib.lbq_lora_workspace_bytes(B(d), 0, 16) == 0
    args = lambda r=16, ws=FAKE, wsb=need, A=FAKE, Bm=FAKE, sigma=1.0: lib.lbq_lora_fwd(
        B(d), B(q), FAKE, 8, A, Bm, r, sigma, FAKE, 64, ws, wsb, None)
    assert _status(L, args(r=0)) == "LBQ_E_SHAPE"
    assert _status(L, args(r=65)) == "LBQ_E_SHAPE"
    assert _status(L, args(ws=None)) == "LBQ_E_WORKSPACE"
    assert _status(L, args(wsb=need - 1)) == "LBQ_E_WORKSPACE"
    assert _status(L, args(A=None)) == "LBQ_E_NULL"
    assert _status(L, args(A=FAKE + 2)) == "LBQ_E_ALIGN"
    assert _status(L, args(Bm=FAKE + 1)) == "LBQ_E_ALIGN"
    assert _status(L, args(sigma=float("inf"))) == "LBQ_E_SHAPE"
    assert _status(L, args(ws=FAKE + 8)) == "LBQ_E_ALIGN"


def test_grouped_fwd_error_paths(L):
    lib = L.lib
    import re
    hdr = open(L._lib.HERE + "/../include/lbq.h").read()
    assert int(re.search(r"#define LBQ_MAX_GROUP (\d+)", hdr).group(1)) == L.LBQ_MAX_GROUP
    d = [L.make_desc("minmax", 64, 256), L.make_desc("minmax", 32, 256, 2, 64), L.make_desc("nf4", 128, 256, double_quant=True)]

    def call(descs=d, qs=None, X=FAKE, m=1, ys=None, ldys=None, ws=None, wsb=0, count=None):
        c = len(descs) if count is None else count
        D = (L.Desc * len(descs))(*descs)
        Q = (L.QTensor * len(descs))(*(qs or [_q(L) for _ in descs]))
        Y = (ctypes.c_void_p * len(descs))(*(ys or [FAKE] * len(descs)))
        LD = (ctypes.c_int64 * len(descs))(*(ldys or [x.n for x in descs]))
        return _status(L, lib.lbq_linear_fwd_grouped(c, D, Q, X, m, Y, LD, ws, wsb, None))

    assert call(count=0) == "LBQ_E_SHAPE"
    assert call(descs=d * 3) == "LBQ_E_SHAPE"  # 9 > LBQ_MAX_GROUP
    assert _status(L, lib.lbq_linear_fwd_grouped(1, None, None, FAKE, 1, None, None, None, 0, None)) == "LBQ_E_NULL"
    assert call(descs=[d[0], L.make_desc("minmax", 64, 512)]) == "LBQ_E_SHAPE"  # k differs
    assert call(X=FAKE + 8) == "LBQ_E_ALIGN"
    assert call(ys=[FAKE, FAKE + 1, FAKE]) == "LBQ_E_ALIGN"  # weight 1's Y
    assert call(ldys=[64, 31, 128]) == "LBQ_E_SHAPE"  # weight 1's ldy < n
    assert call(m=0) == "LBQ_OK"  # empty batch: nothing enqueued
    # a K split at m = 16 needs fp32 partials: the largest of the weights' workspaces
    dk = [L.make_desc("minmax", 64, 8192), L.make_desc("nf4", 1024, 8192, double_quant=True)]
    D = (L.Desc * 2)(*dk)
    need = lib.lbq_linear_fwd_grouped_workspace_bytes(2, D, 16)
    assert need == max(lib.lbq_linear_workspace_bytes(ctypes.byref(x), 16) for x in dk) > 0
    assert lib.lbq_linear_fwd_grouped_workspace_bytes(2, D, 1) == 0
    assert lib.lbq_linear_fwd_grouped_workspace_bytes(0, D, 16) == 0
    assert call(descs=dk, m=16, ws=None, wsb=0) == "LBQ_E_WORKSPACE"
    assert call(descs=dk, m=16, ws=FAKE, wsb=need - 1) == "LBQ_E_WORKSPACE"
    assert call(descs=dk, m=16, ws=FAKE + 8, wsb=need) == "LBQ_E_ALIGN"


def test_gemm_split_workspace_sizes(L):
    """For m > 64 the workspace queries report the GEMM's K-split partials,
    ks * m * n fp32 per weight, when a weight's 256x256 output tiles fill at
    most half the chip: ks up to 256 / tiles, at most 8 and at most k / 3200
    in 1024-code ranges (k / 512 in 512-code ranges for m <= 256 and at most
    32 tiles), then the count of non-empty ranges; 0 when the
    tiles fill the chip or K is short.  The grouped query takes the largest
    kind group's sum.  A call with less (here: none) runs the GEMM unsplit,
    so no error."""
    lib, B = L.lib, ctypes.byref
    ws = lambda d, m: lib.lbq_linear_workspace_bytes(B(d), m)
    d8k = L.make_desc("minmax", 1024, 8192)
    assert ws(d8k, 257) == 2 * 257 * 1024 * 4              # 8 tiles; k / 3200 = 2
    assert ws(L.make_desc("minmax", 2048, 28672), 1024) == 7 * 1024 * 2048 * 4  # 32 tiles: 8 ranges of 3584 -> 7 of 4096
    assert ws(L.make_desc("minmax", 4096, 4096), 128) == 8 * 128 * 4096 * 4    # m <= 256, 16 tiles: 512-code ranges
    assert ws(L.make_desc("minmax", 4096, 1536), 100) == 3 * 100 * 4096 * 4    # k / 512 = 3
    assert ws(L.make_desc("minmax", 14336, 4096), 128) == 0                    # 56 tiles: k / 3200 = 1
    assert ws(L.make_desc("minmax", 4096, 4096), 4096) == 0   # 256 tiles fill the chip
    assert ws(L.make_desc("minmax", 4096, 14336), 2048) == 2 * 2048 * 4096 * 4  # 128 tiles: half the chip
    assert ws(L.make_desc("minmax", 4096, 14336), 2304) == 0  # 144 tiles
    assert ws(L.make_desc("minmax", 1024, 4096), 257) == 0    # k / 3200 = 1
    assert ws(L.make_desc("nf4", 8192, 49152, double_quant=True), 512) == 4 * 512 * 8192 * 4  # 64 tiles: 256 / 64
    dk = [d8k, L.make_desc("minmax", 512, 8192), L.make_desc("minmax", 256, 8192, bits=2)]
    D = (L.Desc * 3)(*dk)
    i4 = ws(dk[0], 130) + ws(dk[1], 130)
    assert lib.lbq_linear_fwd_grouped_workspace_bytes(3, D, 130) == max(i4, ws(dk[2], 130)) > 0


def test_grouped_bwd_error_paths(L):
    lib = L.lib
    d = [L.make_desc("minmax", 64, 256), L.make_desc("minmax", 128, 256), L.make_desc("minmax", 32, 256)]

    def call(descs=d, dys=None, dX=FAKE, m=4, count=None):
        c = len(descs) if count is None else count
        D = (L.Desc * len(descs))(*descs)
        Q = (L.QTensor * len(descs))(*[_q(L) for _ in descs])
        P = (ctypes.c_void_p * len(descs))(*(dys or [FAKE] * len(descs)))
        return _status(L, lib.lbq_linear_bwd_dx_grouped(c, D, Q, P, m, dX, None))

    assert call(count=0) == "LBQ_E_SHAPE"
    assert call(descs=d * 3) == "LBQ_E_SHAPE"  # 9 > LBQ_MAX_GROUP
    assert _status(L, lib.lbq_linear_bwd_dx_grouped(1, None, None, None, 4, FAKE, None)) == "LBQ_E_NULL"
    assert call(descs=[d[0], L.make_desc("minmax", 64, 512)]) == "LBQ_E_SHAPE"  # k differs
    assert call(descs=[d[0], L.make_desc("minmax", 64, 256, 2, 64)]) == "LBQ_E_UNSUPPORTED"  # formats differ
    assert call(descs=[d[0], L.make_desc("minmax", 60, 256)]) == "LBQ_E_SHAPE"  # n % 8 != 0
    assert call(dys=[FAKE, FAKE + 8, FAKE]) == "LBQ_E_ALIGN"  # weight 1's dY
    assert call(dX=FAKE + 8) == "LBQ_E_ALIGN"
    assert call(m=0) == "LBQ_OK"  # empty batch: nothing enqueued


def test_lora_bwd_error_paths(L):
    lib = L.lib
    B = ctypes.byref
    d = L.make_desc("nf4", 64, 256, double_quant=True)
    q = _q(L)
    need = lib.lbq_lora_bwd_workspace_bytes(B(d), 8, 16)
    # B^T [32][n] + G and T [m][32] bf16, then fp32 partials of at least [16][max(n, k)]
    assert need >= 32 * 64 * 2 + 2 * 8 * 32 * 2 + 16 * 256 * 4 and need % 16 == 0
    assert lib.lbq_lora_bwd_workspace_bytes(B(d), 0, 16) == 0
    assert lib.lbq_lora_bwd_workspace_bytes(B(d), 8, 65) == 0

    def args(m=8, r=16, ws=FAKE, wsb=need, X=FAKE, A=FAKE, Bm=FAKE, dA=FAKE, dB=FAKE, sigma=1.0, desc=d):
        return lib.lbq_lora_bwd(B(desc), B(q), X, FAKE, m, A, Bm, r, sigma, FAKE, dA, dB, ws, wsb, None)

    assert _status(L, args(r=0)) == "LBQ_E_SHAPE"
    assert _status(L, args(r=65)) == "LBQ_E_SHAPE"
    assert _status(L, args(sigma=float("nan"))) == "LBQ_E_SHAPE"
    assert _status(L, args(A=None)) == "LBQ_E_NULL"
    assert _status(L, args(dB=None)) == "LBQ_E_NULL"
    assert _status(L, args(X=None)) == "LBQ_E_NULL"
    assert _status(L, args(X=FAKE + 8)) == "LBQ_E_ALIGN"
    assert _status(L, args(A=FAKE + 2)) == "LBQ_E_ALIGN"
    assert _status(L, args(Bm=FAKE + 1)) == "LBQ_E_ALIGN"
    assert _status(L, args(dA=FAKE + 2)) == "LBQ_E_ALIGN"
    assert _status(L, args(ws=None)) == "LBQ_E_WORKSPACE"
    assert _status(L, args(wsb=need - 1)) == "LBQ_E_WORKSPACE"
    assert _status(L, args(ws=FAKE + 8)) == "LBQ_E_ALIGN"
    d96 = L.make_desc("nf4", 96, 256, double_quant=True)  # n % 64 != 0
    need96 = lib.lbq_lora_bwd_workspace_bytes(B(d96), 8, 16)
    assert _status(L, args(desc=d96, wsb=need96)) == "LBQ_E_SHAPE"
    assert _status(L, lib.lbq_lora_bwd(B(d), B(_q(L, out_rows=FAKE)), FAKE, FAKE, 8, FAKE, FAKE, 16, 1.0,
                                       FAKE, FAKE, FAKE, FAKE, need, None)) == "LBQ_E_UNSUPPORTED"


def test_blob_header_and_error_paths(L):
    """The blob layout as lbq.h documents it, built by hand here (no device
    access: every path below fails or finishes before any copy)."""
    import struct
    lib = L.lib
    B = ctypes.byref
    for args in (("minmax", 3, 384, 4, 128), ("minmax", 5, 256, 2, 64), ("nf4", 7, 512)):
        d = L.make_desc(*args) if args[0] == "minmax" else L.make_desc(*args, double_quant=True)
        sz = L.lbq_layout(d)
        keys = ("packed", "scales", "zeros", "absmax", "absmax_q", "absmax_scale")
        total = 96 + sum((sz[k] + 15) // 16 * 16 for k in keys)
        assert lib.lbq_serialized_bytes(B(d)) == total
        hdr = b"LBQ1" + struct.pack("<I", 1) + bytes(d) + struct.pack("<6Q", *[sz[k] for k in keys])
        assert len(hdr) == 96
        blob = hdr + bytes(total - 96)
        out = L.Desc()
        assert _status(L, lib.lbq_blob_desc(blob, len(blob), B(out))) == "LBQ_OK"
        assert bytes(out) == bytes(d)
        assert _status(L, lib.lbq_blob_desc(b"LBQ2" + blob[4:], len(blob), B(out))) == "LBQ_E_FORMAT"
        assert _status(L, lib.lbq_blob_desc(blob[:4] + struct.pack("<I", 2) + blob[8:], len(blob), B(out))) == "LBQ_E_FORMAT"
        assert _status(L, lib.lbq_blob_desc(blob, len(blob) - 1, B(out))) == "LBQ_E_SHAPE"
        assert _status(L, lib.lbq_blob_desc(blob, 95, B(out))) == "LBQ_E_SHAPE"
        wrong = hdr[:48] + struct.pack("<Q", sz["packed"] + 16) + hdr[56:]
        assert _status(L, lib.lbq_blob_desc(wrong + blob[96:], len(blob), B(out))) == "LBQ_E_FORMAT"
        bad = L.make_desc("minmax", 3, 384)
        bad.bits = 3
        assert _status(L, lib.lbq_blob_desc(hdr[:8] + bytes(bad) + hdr[48:] + blob[96:], len(blob), B(out))) == "LBQ_E_FORMAT"
        assert _status(L, lib.lbq_blob_desc(None, len(blob), B(out))) == "LBQ_E_NULL"
        # checks that stop before any copy
        assert _status(L, lib.lbq_serialize(B(d), B(_q(L)), blob, total - 1, None)) == "LBQ_E_SHAPE"
        assert _status(L, lib.lbq_serialize(B(d), B(_q(L)), None, total, None)) == "LBQ_E_NULL"
        assert _status(L, lib.lbq_deserialize(blob, len(blob), B(_q(L, packed=None)), None)) == "LBQ_E_NULL"
        assert _status(L, lib.lbq_deserialize(b"XBQ1" + blob[4:], len(blob), B(_q(L)), None)) == "LBQ_E_FORMAT"
    assert lib.lbq_serialized_bytes(B(L.make_desc("minmax", 0, 256))) == 0


def test_strerror_covers_every_status(L):
    for code in range(8):
        assert L.lib.lbq_strerror(code).decode() not in ("", "unknown status")
    assert L.lib.lbq_strerror(99).decode() == "unknown status"
