"""CPU oracle for group-wise low-bit weight quantization and the dequantize-then-matmul.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, table or
constant generator with the HIP library; the only thing both sides read is the
seeded input module ``synth_inputs``.

It is written to be read against the pages, step by step, in plain numpy:

* fp32 quantization arithmetic is done with numpy float32 elementwise ops,
  each of which is one IEEE-754 binary32 operation rounded to nearest-even
  (true division, no fused multiply-add);
* integer rounding is ``numpy.rint`` (round half to even);
* matmuls accumulate in fp64 with numpy's fp64 ``matmul`` over operands that
  are exact in fp64.

Sources (cited by page title and section):
  [GB]  GreenBit.AI, "只需单卡RTX 3090，低比特量化训练就能实现LLaMA-3 8B全参微调",
        section 模型量化 (model quantization): the classic group-wise MinMax
        quantizer, INT4 with group size 128 and INT2 with group size 64 as the
        only base representations, round-to-nearest.
  [BNB] bitsandbytes FSDP-QLoRA guide (walk-through of docs/source/fsdp_qlora.md),
        section 量化数据的存储 (storing quantized data): two 4-bit codes per
        byte, even-indexed code in the high nibble; section 通过BitsAndBytesConfig配置:
        weights are unpacked and dequantized to the compute dtype (bf16) inside
        the kernel; parameter table of step 2: nf4, double quant of the absmax.
  [QL]  "QLoRA技术在量化微调中的应用", section QLoRA技术原理: NF4 is a 4-bit
        NormalFloat type built for normally distributed weights; double
        quantization quantizes the quantization constants and saves about
        0.37 bit per parameter; gradients flow through the frozen 4-bit model
        into low-rank adapters.

Readings where the pages are silent:
  * MinMax is asymmetric with an integer zero point; the group range always
    includes 0 (lo = min(0, min w), hi = max(0, max w)); a scale that comes
    out as 0 (an all-zero group) is replaced by 1.
  * Groups run along K (the input dimension), contiguous, K % g == 0.
  * 2-bit codes are packed four per byte, first code in the two high bits.
  * NF4 levels: 8 positive normal quantiles at evenly spaced probabilities
    from delta = 1 - (1/30 + 1/32)/2 down to 1/2 (last one dropped), 7 negative
    ones likewise from 8 points, plus an exact 0, normalised to [-1, 1];
    computed in fp64, rounded once to fp32.  Encoding is the nearest level by
    the fp32 midpoint rule (a tie goes to the lower code).
  * Double quantization: blocks of 256 consecutive absmax values, symmetric
    int8 codes 0..127 with an fp32 second-level scale c2 = max/127; the 4-bit
    codes are computed from the un-quantized absmax.
  * Dequantized weights are rounded to bf16 (round to nearest-even) from one
    fp32 product.

Every function below is pinned by tests/test_oracle_pins.py to facts the pages
and plain mathematics fix (packing vectors, closed forms, brute-force searches,
invariants).  No function is "parity unpinned".
"""
from __future__ import annotations

import math
from statistics import NormalDist

import numpy as np

F32 = np.float32

# --------------------------------------------------------------------------
# bf16 (round to nearest-even) -- the compute dtype of [BNB] §通过BitsAndBytesConfig配置
# --------------------------------------------------------------------------


def bf16_bits(x) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even.

    Keep the top 16 bits of the binary32 pattern after adding 0x7FFF plus the
    lowest kept bit.  (NaN inputs are outside the contract.)"""
    u = np.ascontiguousarray(x, dtype=F32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns -> exact fp64 values."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(F32).astype(np.float64)


# --------------------------------------------------------------------------
# Packing ([BNB] §量化数据的存储)
# --------------------------------------------------------------------------


def pack_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    """Pack integer codes along the last axis, 8/bits codes per byte.

    The first (even-indexed) code of each byte lands in the most significant
    bits: for 4-bit codes byte = code[2i]*16 + code[2i+1]; for 2-bit codes the
    same order extended to four crumbs."""
    per = 8 // bits
    c = np.asarray(codes, dtype=np.uint8)
    lead = c.shape[:-1]
    c = c.reshape(lead + (c.shape[-1] // per, per))
    out = np.zeros(c.shape[:-1], dtype=np.uint8)
    for j in range(per):
        out |= (c[..., j] << np.uint8(8 - bits * (j + 1))).astype(np.uint8)
    return out


def unpack_codes(packed: np.ndarray, bits: int) -> np.ndarray:
    """Inverse of :func:`pack_codes`."""
    per = 8 // bits
    p = np.asarray(packed, dtype=np.uint8)
    mask = np.uint8((1 << bits) - 1)
    parts = [(p >> np.uint8(8 - bits * (j + 1))) & mask for j in range(per)]
    return np.stack(parts, axis=-1).reshape(p.shape[:-1] + (p.shape[-1] * per,))


# --------------------------------------------------------------------------
# Group-wise MinMax quantizer, asymmetric RTN ([GB] §模型量化)
# --------------------------------------------------------------------------


def minmax_quantize(W: np.ndarray, bits: int, group: int):
    """Quantize fp32 W[N, K] group by group along K.

    Returns (codes u8[N,K], scales f32[N,K/g], zeros u8[N,K/g]).

    For each group of g consecutive weights of a row:
      lo = min(0, min w), hi = max(0, max w)
      s  = fl(fl(hi - lo) / Qmax)              (s := 1 if it comes out 0)
      z  = clamp(rne(fl(-lo / s)), 0, Qmax)
      q  = clamp(rne(fl(w / s)) + z, 0, Qmax)
    """
    W = np.ascontiguousarray(W, dtype=F32)
    N, K = W.shape
    assert K % group == 0
    qmax = (1 << bits) - 1
    Wg = W.reshape(N, K // group, group)
    lo = np.minimum(F32(0.0), Wg.min(axis=2))
    hi = np.maximum(F32(0.0), Wg.max(axis=2))
    s = (hi - lo) / F32(qmax)
    s = np.where(s == F32(0.0), F32(1.0), s).astype(F32)
    z = np.clip(np.rint(-lo / s), 0, qmax).astype(np.int32)
    r = np.rint(Wg / s[:, :, None]).astype(np.int32)
    q = np.clip(r + z[:, :, None], 0, qmax)
    return q.reshape(N, K).astype(np.uint8), s, z.astype(np.uint8)


def minmax_dequant_bf16(codes, scales, zeros, group: int) -> np.ndarray:
    """bf16 bits of fl((q - z) * s): the kernel-side dequantization to the compute dtype."""
    N, K = codes.shape
    q = codes.reshape(N, K // group, group).astype(np.int32)
    d = (q - zeros.astype(np.int32)[:, :, None]).astype(F32)
    w = d * scales.astype(F32)[:, :, None]
    return bf16_bits(w.reshape(N, K))


def minmax_exact(codes, scales, zeros, group: int) -> np.ndarray:
    """fp64 (q - z) * s, exact (a small integer times an fp32 value)."""
    N, K = codes.shape
    q = codes.reshape(N, K // group, group).astype(np.float64)
    d = q - zeros.astype(np.float64)[:, :, None]
    return (d * scales.astype(np.float64)[:, :, None]).reshape(N, K)


# --------------------------------------------------------------------------
# NF4 with blockwise absmax ([QL] §QLoRA技术原理, [BNB] step-2 parameter table)
# --------------------------------------------------------------------------


def nf4_codebook() -> np.ndarray:
    """The 16 NF4 levels as fp32, ascending, c[0] = -1, c[7] = 0, c[15] = 1.

    Normal quantiles at evenly spaced probabilities: 9 points from delta down
    to 1/2 (the last, the median, dropped) give 8 positive levels; 8 points
    give 7 negative levels; an exact zero is added; all are divided by the
    largest quantile so the extremes are +-1.  fp64 throughout, one rounding
    to fp32 at the end."""
    nd = NormalDist()
    delta = 1.0 - 0.5 * (1.0 / 30.0 + 1.0 / 32.0)
    pos = [nd.inv_cdf(delta + (0.5 - delta) * i / 8.0) for i in range(8)]
    neg = [-nd.inv_cdf(delta + (0.5 - delta) * i / 7.0) for i in range(7)]
    top = nd.inv_cdf(delta)
    levels = sorted(pos + neg + [0.0])
    return np.array([v / top for v in levels], dtype=np.float64).astype(F32)


def nf4_midpoints(c: np.ndarray) -> np.ndarray:
    """fp32 midpoints m_i = fl(fl(c_i + c_{i+1}) * 0.5), i = 0..14."""
    c = np.asarray(c, dtype=F32)
    return ((c[:-1] + c[1:]) * F32(0.5)).astype(F32)


def nf4_quantize(W: np.ndarray, block: int = 64):
    """NF4-encode fp32 W[N, K] in blocks of ``block`` consecutive entries
    (row-major, K % block == 0).

    Returns (codes u8[N,K], absmax f32[N*K/block]).
      a = max |w| over the block; codes are 7 (the zero level) if a == 0;
      otherwise x = fl(w / a) and code = number of midpoints strictly below x.
    """
    W = np.ascontiguousarray(W, dtype=F32)
    N, K = W.shape
    assert K % block == 0
    blocks = W.reshape(-1, block)
    a = np.abs(blocks).max(axis=1).astype(F32)
    safe = np.where(a == F32(0.0), F32(1.0), a)
    x = blocks / safe[:, None]
    mids = nf4_midpoints(nf4_codebook())
    codes = np.searchsorted(mids, x, side="left").astype(np.uint8)
    codes[a == F32(0.0)] = 7
    return codes.reshape(N, K), a


def double_quant(absmax: np.ndarray, block: int = 256):
    """Second-level quantization of the absmax constants ([QL] §QLoRA技术原理).

    Blocks of ``block`` consecutive absmax values (the last may be partial):
      c2 = fl(max / 127); q2 = clamp(rne(fl(a / c2)), 0, 127), q2 = 0 if c2 == 0.
    Returns (absmax_q i8[nb], absmax_scale f32[ceil(nb/block)])."""
    a = np.asarray(absmax, dtype=F32)
    nb = a.shape[0]
    nblk = -(-nb // block)
    q2 = np.zeros(nb, dtype=np.int8)
    c2 = np.zeros(nblk, dtype=F32)
    for b in range(nblk):
        seg = a[b * block:(b + 1) * block]
        c = seg.max() / F32(127.0)
        c2[b] = c
        if c != F32(0.0):
            q2[b * block:(b + 1) * block] = np.clip(np.rint(seg / c), 0, 127).astype(np.int8)
    return q2, c2


def double_dequant_absmax(absmax_q, absmax_scale, block: int = 256) -> np.ndarray:
    """fp32 A_hat = fl(q2 * c2)."""
    q2 = np.asarray(absmax_q, dtype=np.int8).astype(F32)
    c2 = np.repeat(np.asarray(absmax_scale, dtype=F32), block)[: q2.shape[0]]
    return (q2 * c2).astype(F32)


def nf4_dequant_bf16(codes, absmax_f32, block: int = 64) -> np.ndarray:
    """bf16 bits of fl(c[code] * a) with a the (possibly double-dequantized) absmax."""
    N, K = codes.shape
    c = nf4_codebook()
    vals = c[codes.reshape(-1, block)] * np.asarray(absmax_f32, dtype=F32)[:, None]
    return bf16_bits(vals.astype(F32).reshape(N, K))


def nf4_exact(codes, absmax_f32, block: int = 64) -> np.ndarray:
    """fp64 c[code] * a, exact (product of two fp32 values)."""
    N, K = codes.shape
    c = nf4_codebook().astype(np.float64)
    a = np.asarray(absmax_f32, dtype=F32).astype(np.float64)
    return (c[codes.reshape(-1, block)] * a[:, None]).reshape(N, K)


# --------------------------------------------------------------------------
# Sizes and the double-quantization saving ([QL] §QLoRA技术原理)
# --------------------------------------------------------------------------


def nf4_metadata_bytes(n: int, k: int, double_quant_on: bool, block: int = 64,
                       dq_block: int = 256) -> int:
    nb = n * k // block
    if not double_quant_on:
        return 4 * nb
    return nb + 4 * (-(-nb // dq_block))


def dq_saving_bits_per_param(n: int, k: int) -> float:
    """Bits per parameter saved by double quantization, from the byte counts."""
    saved = nf4_metadata_bytes(n, k, False) - nf4_metadata_bytes(n, k, True)
    return 8.0 * saved / (n * k)


# --------------------------------------------------------------------------
# The frozen low-bit linear layer: forward, input gradient, LoRA, channel mix
# --------------------------------------------------------------------------


def linear_fwd(X_bits: np.ndarray, W_exact: np.ndarray) -> np.ndarray:
    """Y = X . W^T in fp64 (X given as bf16 bits [M, K], W exact fp64 [N, K])."""
    return bf16_to_f64(X_bits) @ W_exact.T


def linear_bwd_dx(dY_bits: np.ndarray, W_exact: np.ndarray) -> np.ndarray:
    """dX = dY . W in fp64 ([QL]: gradients pass through the frozen quantized
    weights to reach the adapters)."""
    return bf16_to_f64(dY_bits) @ W_exact


def linear_bwd_dx_grouped(dY_bits_list, W_exact_list) -> np.ndarray:
    """dX = sum_i dY_i . W_i in fp64 for linears that read the same X (the
    chain rule sums the gradients that reach a shared input; [QL]: each passes
    through its frozen quantized weight)."""
    return sum(bf16_to_f64(d) @ W for d, W in zip(dY_bits_list, W_exact_list))


def lora_fwd(X_bits, W_exact, A_bits, B_bits, sigma: float) -> np.ndarray:
    """Y = X . W^T + sigma * (X . A^T) . B^T in fp64; A is [r, K], B is [N, r]."""
    X = bf16_to_f64(X_bits)
    T = X @ bf16_to_f64(A_bits).T
    return X @ W_exact.T + float(sigma) * (T @ bf16_to_f64(B_bits).T)


def lora_bwd(X_bits, dY_bits, W_exact, A_bits, B_bits, sigma: float):
    """Gradients of Y = X . W^T + sigma * (X . A^T) . B^T for a frozen W, in
    fp64 ("QLoRA技术在量化微调中的应用", section QLoRA技术原理: the gradient
    passes through the frozen quantized weight into the low-rank adapters):

        dX = dY . W + sigma * (dY . B) . A      [m, K]
        dA = sigma * (dY . B)^T . X             [r, K]
        dB = sigma * dY^T . (X . A^T)           [N, r]
    """
    X = bf16_to_f64(X_bits)
    dY = bf16_to_f64(dY_bits)
    A = bf16_to_f64(A_bits)
    B = bf16_to_f64(B_bits)
    G = float(sigma) * (dY @ B)
    dX = dY @ W_exact + G @ A
    dA = G.T @ X
    dB = float(sigma) * (dY.T @ (X @ A.T))
    return dX, dA, dB


def channel_mix_fwd(X_bits, parts) -> np.ndarray:
    """Channel-mix forward: ``parts`` is a list of (out_rows int[n_i], W_exact
    [n_i, K]); output channel out_rows[j] of Y takes row j of W_i."""
    X = bf16_to_f64(X_bits)
    n_total = sum(len(r) for r, _ in parts)
    Y = np.zeros((X.shape[0], n_total))
    for rows, We in parts:
        Y[:, rows] = X @ We.T
    return Y


# --------------------------------------------------------------------------
# Convenience: quantize a weight to the full set of stored arrays
# --------------------------------------------------------------------------


def quantize(W: np.ndarray, fmt: str, bits: int = 4, group: int | None = None,
             double_quant_on: bool = True, dq_block: int = 256) -> dict:
    """Return every stored array for ``fmt`` in {'minmax', 'nf4'} plus the
    fp64 exact dequantized weight (``w_exact``) and the bf16 dequant bits.
    ``group`` defaults to 128 for MinMax and to the NF4 absmax block of 64."""
    N, K = W.shape
    if group is None:
        group = 128 if fmt == "minmax" else 64
    out: dict = {}
    if fmt == "minmax":
        codes, s, z = minmax_quantize(W, bits, group)
        out.update(codes=codes, scales=s, zeros=z, packed=pack_codes(codes, bits))
        out["w_exact"] = minmax_exact(codes, s, z, group)
        out["w_bf16"] = minmax_dequant_bf16(codes, s, z, group)
    elif fmt == "nf4":
        codes, a = nf4_quantize(W, group)
        out.update(codes=codes, packed=pack_codes(codes, 4))
        if double_quant_on:
            q2, c2 = double_quant(a, dq_block)
            ahat = double_dequant_absmax(q2, c2, dq_block)
            out.update(absmax_q=q2, absmax_scale=c2, absmax_hat=ahat)
        else:
            ahat = a
            out.update(absmax=a)
        out["w_exact"] = nf4_exact(codes, ahat, group)
        out["w_bf16"] = nf4_dequant_bf16(codes, ahat, group)
    else:
        raise ValueError(fmt)
    return out


def rel_errors(Y: np.ndarray, Y_ref: np.ndarray):
    """(relative Frobenius error, max-abs error / max|Y_ref|)."""
    Y = np.asarray(Y, dtype=np.float64)
    d = Y - Y_ref
    nref = math.sqrt(float((Y_ref * Y_ref).sum()))
    mref = float(np.abs(Y_ref).max()) if Y_ref.size else 0.0
    fro = math.sqrt(float((d * d).sum())) / nref if nref > 0 else math.sqrt(float((d * d).sum()))
    mx = float(np.abs(d).max()) / mref if mref > 0 else float(np.abs(d).max()) if d.size else 0.0
    return fro, mx


# --------------------------------------------------------------------------
# Format variants: compact MinMax metadata, and double quantization with an
# offset.  Neither is spelled out on the pages; each function states the
# reading it implements.
# --------------------------------------------------------------------------


def fp16_round_up(s) -> np.ndarray:
    """The smallest fp16 value >= s for positive fp32 s (round toward +inf),
    saturating at the largest finite fp16, 65504."""
    s = np.asarray(s, dtype=F32)
    with np.errstate(over="ignore"):                # values above 65504 saturate below
        h = s.astype(np.float16)                   # round to nearest-even
        below = h.astype(F32) < s
        h = np.where(below, np.nextafter(h, np.float16(np.inf)), h).astype(np.float16)
    return np.minimum(h, np.float16(65504.0))


def minmax_quantize_compact(W: np.ndarray, bits: int, group: int):
    """Group-wise MinMax RTN ([GB] §模型量化) with compact metadata: an fp16
    scale and the integer zero point, both derived from the stored scale.

    Returns (codes u8[N,K], scales f16[N,K/g], zeros u8[N,K/g]).
      lo, hi, s32 as in :func:`minmax_quantize` (s32 := 1 if it comes out 0);
      s  = fp16_round_up(s32)    (rounding up keeps Qmax * s >= hi - lo)
      z  = clamp(rne(fl(-lo / s)), 0, Qmax)
      q  = clamp(rne(fl(w / s)) + z, 0, Qmax)
    """
    W = np.ascontiguousarray(W, dtype=F32)
    N, K = W.shape
    assert K % group == 0
    qmax = (1 << bits) - 1
    Wg = W.reshape(N, K // group, group)
    lo = np.minimum(F32(0.0), Wg.min(axis=2))
    hi = np.maximum(F32(0.0), Wg.max(axis=2))
    s32 = (hi - lo) / F32(qmax)
    s32 = np.where(s32 == F32(0.0), F32(1.0), s32).astype(F32)
    s16 = fp16_round_up(s32)
    s = s16.astype(F32)
    z = np.clip(np.rint(-lo / s), 0, qmax).astype(np.int32)
    r = np.rint(Wg / s[:, :, None]).astype(np.int32)
    q = np.clip(r + z[:, :, None], 0, qmax)
    return q.reshape(N, K).astype(np.uint8), s16, z.astype(np.uint8)


def fp32_tree_sum(a) -> np.float32:
    """Sum of fp32 values over the binary tree of adjacent pairs in index
    order: the array is padded with zeros to a power of two and each level
    adds elements 2i and 2i+1 with one fp32 addition."""
    v = np.asarray(a, dtype=F32).ravel()
    size = 1
    while size < v.shape[0]:
        size *= 2
    v = np.concatenate([v, np.zeros(size - v.shape[0], dtype=F32)])
    while v.shape[0] > 1:
        v = (v[0::2] + v[1::2]).astype(F32)
    return F32(v[0]) if v.shape[0] else F32(0.0)


def absmax_offset(absmax) -> np.float32:
    """Per-tensor offset of double quantization with an offset: the mean of
    the absmax values, fp32(fp64(tree sum) / nb).  ([QL] §结论 says double
    quantization re-quantizes the scale factor and the offset; [BNB] §源码纵深
    lists `offset` among the quantization-state fields.)"""
    a = np.asarray(absmax, dtype=F32)
    return F32(np.float64(fp32_tree_sum(a)) / np.float64(a.shape[0]))


def double_quant_offset(absmax: np.ndarray, block: int = 256):
    """Double quantization with an offset: the absmax values minus their
    per-tensor mean are quantized to symmetric int8 codes in blocks of
    ``block`` consecutive values with an fp32 scale per block:
      off = absmax_offset(A);  d = fl(A - off)
      c2  = fl(max |d| / 127);  q2 = clamp(rne(fl(d / c2)), -127, 127)  (0 if c2 == 0)
    Returns (absmax_q i8[nb], absmax_scale f32[ceil(nb/block)], offset f32)."""
    a = np.asarray(absmax, dtype=F32)
    nb = a.shape[0]
    off = absmax_offset(a)
    d = (a - off).astype(F32)
    nblk = -(-nb // block)
    q2 = np.zeros(nb, dtype=np.int8)
    c2 = np.zeros(nblk, dtype=F32)
    for b in range(nblk):
        seg = d[b * block:(b + 1) * block]
        c = np.abs(seg).max() / F32(127.0)
        c2[b] = c
        if c != F32(0.0):
            q2[b * block:(b + 1) * block] = np.clip(np.rint(seg / c), -127, 127).astype(np.int8)
    return q2, c2, off


def double_dequant_absmax_offset(absmax_q, absmax_scale, offset, block: int = 256) -> np.ndarray:
    """fp32 A_hat = fl(fl(q2 * c2) + offset)."""
    q2 = np.asarray(absmax_q, dtype=np.int8).astype(F32)
    c2 = np.repeat(np.asarray(absmax_scale, dtype=F32), block)[: q2.shape[0]]
    return ((q2 * c2).astype(F32) + F32(offset)).astype(F32)


def quantize_variant(W: np.ndarray, variant: str) -> dict:
    """Every stored array of a format variant, plus ``w_exact`` (fp64) and
    ``w_bf16`` like :func:`quantize`.
      'i4g128c', 'i2g64c': MinMax with compact metadata; ``scales`` f16,
          ``zeros`` u8 unpacked and ``zeros_packed`` (zero points packed like
          the codes, row by row);
      'nf4dqo': NF4 with double quantization with an offset; ``absmax_q``
          i8, ``absmax_scale`` f32 with the offset appended as one more entry.
    """
    out: dict = {}
    if variant in ("i4g128c", "i2g64c"):
        bits, group = (4, 128) if variant == "i4g128c" else (2, 64)
        codes, s16, z = minmax_quantize_compact(W, bits, group)
        s = s16.astype(F32)
        out.update(codes=codes, scales=s16, zeros=z, zeros_packed=pack_codes(z, bits),
                   packed=pack_codes(codes, bits))
        out["w_exact"] = minmax_exact(codes, s, z, group)
        out["w_bf16"] = minmax_dequant_bf16(codes, s, z, group)
    elif variant == "nf4dqo":
        codes, a = nf4_quantize(W, 64)
        q2, c2, off = double_quant_offset(a, 256)
        ahat = double_dequant_absmax_offset(q2, c2, off, 256)
        out.update(codes=codes, packed=pack_codes(codes, 4), absmax=a, absmax_q=q2,
                   absmax_scale=np.concatenate([c2, np.array([off], dtype=F32)]), absmax_hat=ahat)
        out["w_exact"] = nf4_exact(codes, ahat, 64)
        out["w_bf16"] = nf4_dequant_bf16(codes, ahat, 64)
    else:
        raise ValueError(variant)
    return out


def variant_bits_per_param(variant: str, n: int, k: int) -> float:
    """Stored bits per weight of a format variant, from the byte counts."""
    if variant in ("i4g128c", "i2g64c"):
        bits, group = (4, 128) if variant == "i4g128c" else (2, 64)
        g = k // group
        return 8.0 * (n * k * bits // 8 + n * g * 2 + n * g * bits // 8) / (n * k)
    nb = n * k // 64
    return 8.0 * (n * k // 2 + nb + 4 * (-(-nb // 256) + 1)) / (n * k)
