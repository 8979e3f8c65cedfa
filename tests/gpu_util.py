"""Helpers for the GPU parity tests: move seeded host arrays to the device and
compare device results with the oracle."""
import numpy as np
import torch

from oracle import lbq_oracle as O

DEV = "cuda:0"


def to_dev_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def to_dev_bf16(bits: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.to(DEV).view(torch.bfloat16)


def bf16_bits_host(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy()


def assert_close(Y_bits: np.ndarray, Y_ref: np.ndarray, fro_tol=5e-3, max_tol=2e-2, what=""):
    """The matmul tolerance: relative Frobenius <= 5e-3 and
    max|Y - Y_ref| <= 2e-2 * max|Y_ref|, against the fp64 oracle."""
    Y = O.bf16_to_f64(Y_bits)
    fro, mx = O.rel_errors(Y, Y_ref)
    assert fro <= fro_tol and mx <= max_tol, f"{what}: rel_fro={fro:.3e} max_rel={mx:.3e}"
    return fro, mx


def check_quantized_equal(qw, ref: dict, fmt: str, double_quant: bool = True):
    """Bit-exact comparison of every stored array."""
    assert np.array_equal(host(qw.packed), ref["packed"]), "packed bytes differ"
    if fmt == "minmax":
        s = host(qw.scales).reshape(ref["scales"].shape)
        assert np.array_equal(s.view(np.uint32), ref["scales"].view(np.uint32)), "scales differ"
        assert np.array_equal(host(qw.zeros).reshape(ref["zeros"].shape), ref["zeros"]), "zeros differ"
    elif double_quant:
        assert np.array_equal(host(qw.absmax_q), ref["absmax_q"]), "absmax_q differ"
        assert np.array_equal(host(qw.absmax_scale).view(np.uint32),
                              ref["absmax_scale"].view(np.uint32)), "absmax_scale differ"
    else:
        assert np.array_equal(host(qw.absmax).view(np.uint32), ref["absmax"].view(np.uint32)), "absmax differ"
