"""The allocation-free forward (lbq_linear_fwd_noalloc) against lbq_linear_fwd
with a caller workspace, through the C ABI: the same kernels, so the outputs
must be equal bit for bit, and within the matmul tolerance of the oracle.

Two calls in a row share the library's scratch array; the second, smaller
call must not see anything the first one left there.
"""
import numpy as np
import pytest
import torch

import synth_inputs as SI
from gpu_util import assert_close, bf16_bits_host, to_dev_bf16, to_dev_f32
from oracle import lbq_oracle as O

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    import group_wise_minmax_amd as L
    assert torch.cuda.is_available()
    return L


def _case(L, fmt, bits, group, dq, n, k, m, seed):
    W = SI.gaussian_weights(seed, n, k, outlier_seed=seed + 1)
    X = SI.bf16_normal(seed + 2, (m, k))
    qw = L.lbq_quantize(to_dev_f32(W), fmt, bits, group, dq)
    ref = O.quantize(W, fmt, bits, group, dq)
    return qw, to_dev_bf16(X), O.linear_fwd(X, ref["w_exact"])


# (format, bits, group, dq), then (n, k, m) of the first and the second call:
# the second is smaller in every dimension (or equal in k), and m spans the
# small-batch range that uses the scratch (split K), m = 1 and a GEMM size that
# do not, and GEMMs whose K split uses it.
CASES = [
    (("minmax", 4, 128, False), (4096, 4096, 40), (1040, 1280, 20)),
    (("minmax", 2, 64, False), (2048, 8192, 64), (300, 1024, 16)),
    (("nf4", 4, 64, True), (4096, 4096, 16), (512, 512, 5)),
    (("minmax", 4, 128, False), (32704, 2048, 64), (4096, 2048, 33)),   # the largest scratch any shape needs
    (("minmax", 4, 128, False), (1024, 1024, 1), (256, 256, 130)),
    (("nf4", 4, 64, True), (1024, 8192, 257), (512, 8192, 100)),       # GEMMs that split K
]


@pytest.mark.parametrize("spec,first,second", CASES,
                         ids=["i4g128", "i2g64", "nf4dq", "max_scratch", "gemv_gemm", "gemm_split"])
def test_noalloc_matches_workspace_forward_twice(L, spec, first, second):
    fmt, bits, group, dq = spec
    for call, (n, k, m) in enumerate((first, second)):
        qw, X, Yref = _case(L, fmt, bits, group, dq, n, k, m, 9100 + 10 * call + n % 7)
        Y_ws = L.lbq_linear_fwd(X, qw)
        Y_na = L.lbq_linear_fwd_noalloc(X, qw)
        torch.cuda.synchronize()
        assert torch.equal(Y_na.view(torch.int16), Y_ws.view(torch.int16)), f"call {call}: noalloc != workspace forward"
        assert_close(bf16_bits_host(Y_na), Yref, what=f"call {call} {fmt} n={n} k={k} m={m}")


def test_noalloc_empty_batch_and_errors(L):
    qw = L.lbq_quantize(to_dev_f32(SI.gaussian_weights(9200, 64, 256)), "minmax", 4, 128)
    X = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda:0")
    Y = L.lbq_linear_fwd_noalloc(X, qw)
    assert Y.shape == (0, 64)
    with pytest.raises(L.LbqError) as e:  # a descriptor error is caught before anything runs
        bad = L.make_desc("minmax", 64, 256, 3, 128)
        q = qw.qtensor()
        import ctypes
        from group_wise_minmax_amd._lib import check, lib
        Xg = torch.zeros((4, 256), dtype=torch.bfloat16, device="cuda:0")
        Yg = torch.zeros((4, 64), dtype=torch.bfloat16, device="cuda:0")
        check(lib.lbq_linear_fwd_noalloc(ctypes.byref(bad), ctypes.byref(q), Xg.data_ptr(), 4, Yg.data_ptr(), 64,
                                         None), "lbq_linear_fwd_noalloc")
    assert e.value.name == "LBQ_E_FORMAT"
