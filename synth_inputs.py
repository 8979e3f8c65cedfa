"""Seeded synthetic inputs shared by the oracle-side tests, the GPU tests and bench.py.

This module only draws random numbers and reshapes them; it holds none of the
quantizer's or the matmul's arithmetic.  Every tensor is produced on the host
with numpy's PCG64 (``numpy.random.default_rng``) so that the CPU oracle and the
HIP path read the very same bytes.

Distributions follow the workloads the pages describe:
  * weights ~ N(0, 0.02) with a sparse set of large outliers (0.1 % of entries
    scaled by 20) -- the "systematic outlier channels" remark of the GreenBit.AI
    article (only-one-RTX-3090 LLaMA-3 8B fine-tuning), section 模型量化, and
    the normal-weight premise of NF4 in the QLoRA overview
    ("QLoRA技术在量化微调中的应用", section QLoRA技术原理);
  * heavy-tailed weights (Student-t, nu = 5, rescaled to std 0.015) for the
    Qwen1.5-110B-shaped layer;
  * activations / output gradients ~ N(0, 1) rounded to bf16, LoRA factors
    ~ N(0, 0.01) rounded to bf16.

bf16 rounding of the *inputs* is done by torch's CPU conversion (a library
routine), so this module carries no rounding code of its own.

Seed convention: ``seed = 1000*config + 10*layer_idx + slot`` with slot
0 = W, 1 = outlier mask, 2 = X, 3 = LoRA A, 4 = LoRA B, 5 = dY, 6 = channel mask.
Layer order is q, k, v, o, gate, up, down (idx 0..6).
"""
from __future__ import annotations

import numpy as np

SLOT_W, SLOT_OUTLIER, SLOT_X, SLOT_A, SLOT_B, SLOT_DY, SLOT_CHMASK = range(7)

LAYER_NAMES = ("q", "k", "v", "o", "gate", "up", "down")

# (N, K) = (out, in) of each linear of one decoder layer.
LLAMA3_8B = {
    "q": (4096, 4096), "k": (1024, 4096), "v": (1024, 4096), "o": (4096, 4096),
    "gate": (14336, 4096), "up": (14336, 4096), "down": (4096, 14336),
}
LLAMA3_70B = {
    "q": (8192, 8192), "k": (1024, 8192), "v": (1024, 8192), "o": (8192, 8192),
    "gate": (28672, 8192), "up": (28672, 8192), "down": (8192, 28672),
}
QWEN15_110B = {
    "q": (8192, 8192), "k": (1024, 8192), "v": (1024, 8192), "o": (8192, 8192),
    "gate": (49152, 8192), "up": (49152, 8192), "down": (8192, 49152),
}


def seed_of(config: int, layer_idx: int, slot: int) -> int:
    return 1000 * config + 10 * layer_idx + slot


def gaussian_weights(seed: int, n: int, k: int, std: float = 0.02,
                     outlier_seed: int | None = None, outlier_p: float = 0.001,
                     outlier_mult: float = 20.0) -> np.ndarray:
    """fp32 [n, k] ~ std*N(0,1); if ``outlier_seed`` is given, a Bernoulli(p)
    mask drawn from it multiplies the selected entries by ``outlier_mult``."""
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((n, k), dtype=np.float32)
    w *= np.float32(std)
    if outlier_seed is not None:
        mrng = np.random.default_rng(outlier_seed)
        mask = mrng.random((n, k), dtype=np.float32) < np.float32(outlier_p)
        w[mask] *= np.float32(outlier_mult)
    return w


def student_t_weights(seed: int, n: int, k: int, std: float = 0.015,
                      nu: float = 5.0) -> np.ndarray:
    """fp32 [n, k] Student-t(nu) rescaled to standard deviation ``std``."""
    rng = np.random.default_rng(seed)
    t = rng.standard_t(nu, size=(n, k))
    return (t * (std / np.sqrt(nu / (nu - 2.0)))).astype(np.float32)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 -> bf16 with torch's CPU conversion; return the uint16 bit patterns."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_normal(seed: int, shape, std: float = 1.0) -> np.ndarray:
    """bf16 bit patterns (uint16) of std*N(0,1)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return to_bf16_bits(x)


def bf16_small_ints(seed: int, shape, lo: int = -2, hi: int = 2) -> np.ndarray:
    """bf16 bit patterns of integers drawn uniformly from [lo, hi] (exact in bf16)."""
    rng = np.random.default_rng(seed)
    return to_bf16_bits(rng.integers(lo, hi + 1, size=shape).astype(np.float32))


def channel_mask(seed: int, n: int, frac4: float = 0.25) -> np.ndarray:
    """Sorted int32 indices of the output channels that take the 4-bit format."""
    rng = np.random.default_rng(seed)
    idx = rng.permutation(n)[: int(round(n * frac4))]
    return np.sort(idx).astype(np.int32)


def grid_weights(seed: int, n: int, k: int, group: int, bits: int,
                 exp: int = 4, maxdev: int = 15) -> np.ndarray:
    """Weights that sit exactly on a power-of-two grid, group by group.

    Each group of ``group`` consecutive entries gets an integer offset ``z``
    and integer levels ``c`` in [0, 2^bits-1] (the group always contains both
    0 and 2^bits-1, and c == z occurs), and w = (c - z) * 2^-exp.  Returned
    together with nothing else: the caller derives expectations independently.
    ``maxdev`` bounds |c - z|.
    """
    rng = np.random.default_rng(seed)
    qmax = (1 << bits) - 1
    ng = k // group
    z = rng.integers(0, qmax + 1, size=(n, ng))
    c = rng.integers(0, qmax + 1, size=(n, ng, group))
    c[:, :, 0] = 0
    c[:, :, 1] = qmax
    c[:, :, 2] = z
    dev = np.clip(c - z[:, :, None], -maxdev, maxdev)
    # keep the extremes so the group's range is exactly [-z, qmax-z] * 2^-exp
    dev[:, :, 0] = -z
    dev[:, :, 1] = qmax - z
    perm = rng.permuted(np.broadcast_to(np.arange(group), (n, ng, group)), axis=2)
    dev = np.take_along_axis(dev, perm, axis=2)
    return (dev.astype(np.float64) * 2.0 ** (-exp)).astype(np.float32).reshape(n, k)


# ---------------------------------------------------------------------------
# Device-side generators for full-size layers (bench).  Same recipes as above,
# drawn with torch's seeded device RNG (Philox) so that 0.2-0.9 G-parameter
# layers are produced in milliseconds.  Tests that compare with the oracle copy
# the generated tensor back to the host; nothing here is method arithmetic.
# ---------------------------------------------------------------------------


def dev_gaussian_weights(seed: int, n: int, k: int, device, std: float = 0.02,
                         outlier_p: float = 0.001, outlier_mult: float = 20.0):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    w = torch.randn((n, k), generator=g, device=device, dtype=torch.float32) * std
    if outlier_p > 0:
        mask = torch.rand((n, k), generator=g, device=device) < outlier_p
        w = torch.where(mask, w * outlier_mult, w)
    return w


def dev_student_t_weights(seed: int, n: int, k: int, device, std: float = 0.015, nu: float = 5.0):
    """Student-t(nu) as normal / sqrt(chi2_nu / nu), rescaled to ``std``."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    z = torch.randn((n, k), generator=g, device=device, dtype=torch.float32)
    chi2 = torch.zeros((n, k), device=device, dtype=torch.float32)
    for _ in range(int(nu)):
        chi2 += torch.randn((n, k), generator=g, device=device, dtype=torch.float32) ** 2
    t = z / torch.sqrt(chi2 / nu)
    return t * (std / (nu / (nu - 2.0)) ** 0.5)


def dev_bf16_normal(seed: int, shape, device, std: float = 1.0):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return (torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std).to(torch.bfloat16)


def dev_channel_mask(seed: int, n: int, device, frac4: float = 0.25):
    import torch
    idx = channel_mask(seed, n, frac4)
    return torch.from_numpy(idx).to(device)
