"""group_wise_minmax_amd -- low-bit group-wise weight quantization and the fused
dequantize-then-matmul of a frozen low-bit linear layer on AMD MI355X (gfx950).

This package is a thin binding over the C ABI of ``liblbq.so``
(``include/lbq.h``): every function below only marshals torch tensors into
pointers and sizes, allocates outputs with torch, and calls the library on the
current HIP stream.  All arithmetic runs in the library's HIP kernels; there is
no fallback.  The functions carry the C names:

    lbq_layout, lbq_quantize, lbq_dequant, lbq_linear_fwd, lbq_linear_bwd_dx,
    lbq_lora_fwd, lbq_nf4_codebook

Formats (cited by page title and section):
  * MinMax INT4 g128 / INT2 g64 -- GreenBit.AI, "只需单卡RTX 3090，低比特量化训练
    就能实现LLaMA-3 8B全参微调", section 模型量化;
  * NF4 with optional double quantization of the absmax -- "QLoRA技术在量化微调中的应用",
    section QLoRA技术原理; bitsandbytes FSDP-QLoRA guide, step 2 parameter table.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass, field
from typing import Optional

import torch

from ._lib import (LBQ_MAX_GROUP, LBQ_META_COMPACT, LBQ_META_F32, LBQ_MINMAX, LBQ_NF4, Desc, LbqError, QTensor, Sizes, check, lib,  # noqa: F401
                   STATUS_CODE, EXPORTED, LIB_PATH)

__all__ = [
    "QuantizedWeight", "make_desc", "lbq_layout", "lbq_quantize", "lbq_dequant",
    "lbq_linear_fwd", "lbq_linear_bwd_dx", "lbq_linear_bwd_dx_grouped", "lbq_lora_fwd", "lbq_nf4_codebook",
    "lbq_linear_workspace_bytes", "lbq_lora_workspace_bytes", "LbqError", "version",
]

_FMT = {"minmax": LBQ_MINMAX, "nf4": LBQ_NF4}


def version() -> str:
    return lib.lbq_version().decode()


def make_desc(fmt: str, n: int, k: int, bits: int = 4, group: Optional[int] = None,
              double_quant: bool = True, compact: bool = False, dq_offset: bool = False) -> Desc:
    """Descriptor for W[n][k]. MinMax: bits 4/2, group 128/64 (default 128 for
    4-bit, 64 for 2-bit), ``compact`` for fp16 scales and packed zero points.
    NF4: absmax block 64, optional double quant (256), ``dq_offset`` for
    double quantization with a per-tensor offset."""
    if fmt not in _FMT:
        raise ValueError(f"format must be one of {sorted(_FMT)}")
    d = Desc()
    d.format = _FMT[fmt]
    d.meta = 0
    if fmt == "minmax":
        d.bits = bits
        d.group = group if group is not None else (128 if bits == 4 else 64)
        d.double_quant = 0
        d.dq_block = 0
        d.meta = LBQ_META_COMPACT if compact else LBQ_META_F32
    else:
        d.bits = 4
        d.group = 64 if group is None else group
        d.double_quant = (2 if dq_offset else 1) if double_quant else 0
        d.dq_block = 256 if double_quant else 0
    d.n = n
    d.k = k
    return d


def lbq_layout(desc: Desc) -> dict:
    s = Sizes()
    check(lib.lbq_layout(ctypes.byref(desc), ctypes.byref(s)), "lbq_layout")
    return {f: getattr(s, f) for f, _ in Sizes._fields_}


def lbq_nf4_codebook() -> list:
    buf = (ctypes.c_float * 16)()
    lib.lbq_nf4_codebook(buf)
    return list(buf)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(device: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, shape=None) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


@dataclass
class QuantizedWeight:
    """Device buffers of one quantized weight plus its descriptor."""
    desc: Desc
    packed: torch.Tensor
    scales: Optional[torch.Tensor] = None
    zeros: Optional[torch.Tensor] = None
    absmax: Optional[torch.Tensor] = None
    absmax_q: Optional[torch.Tensor] = None
    absmax_scale: Optional[torch.Tensor] = None
    out_rows: Optional[torch.Tensor] = field(default=None)

    @property
    def n(self) -> int:
        return self.desc.n

    @property
    def k(self) -> int:
        return self.desc.k

    @property
    def device(self) -> torch.device:
        return self.packed.device

    def qtensor(self) -> QTensor:
        q = QTensor()
        q.packed = _ptr(self.packed)
        q.scales = _ptr(self.scales)
        q.zeros = _ptr(self.zeros)
        q.absmax = _ptr(self.absmax)
        q.absmax_q = _ptr(self.absmax_q)
        q.absmax_scale = _ptr(self.absmax_scale)
        q.out_rows = _ptr(self.out_rows)
        return q

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in
                   (self.packed, self.scales, self.zeros, self.absmax, self.absmax_q,
                    self.absmax_scale) if t is not None)

    def to_bytes(self) -> bytes:
        """The weight and its quantization state as one blob (see
        ``lbq_serialize`` in lbq.h); ``out_rows`` is not part of it."""
        nbytes = lib.lbq_serialized_bytes(ctypes.byref(self.desc))
        buf = ctypes.create_string_buffer(nbytes)
        q = self.qtensor()
        check(lib.lbq_serialize(ctypes.byref(self.desc), ctypes.byref(q), buf, nbytes, _stream(self.device)),
              "lbq_serialize")
        return buf.raw

    @staticmethod
    def from_bytes(blob: bytes, device) -> "QuantizedWeight":
        """Rebuild a weight from ``to_bytes`` output into new device buffers."""
        desc = Desc()
        check(lib.lbq_blob_desc(blob, len(blob), ctypes.byref(desc)), "lbq_blob_desc")
        qw = QuantizedWeight.empty(desc, device)
        q = qw.qtensor()
        check(lib.lbq_deserialize(blob, len(blob), ctypes.byref(q), _stream(qw.device)), "lbq_deserialize")
        return qw

    def storage_view(self, dtype: torch.dtype = torch.bfloat16) -> torch.Tensor:
        """The packed bytes reinterpreted as ``dtype`` (same bits, no copy):
        the float storage a sharding framework can hold them in."""
        return self.packed.view(dtype)

    @staticmethod
    def empty(desc: Desc, device) -> "QuantizedWeight":
        sz = lbq_layout(desc)
        dev = torch.device(device)
        n, k = desc.n, desc.k
        qw = QuantizedWeight(desc, torch.empty((n, sz["packed"] // n), dtype=torch.uint8, device=dev))
        if sz["scales"]:
            if desc.meta == LBQ_META_COMPACT:
                qw.scales = torch.empty((n, sz["scales"] // 2 // n), dtype=torch.float16, device=dev)
            else:
                qw.scales = torch.empty((n, sz["scales"] // 4 // n), dtype=torch.float32, device=dev)
            qw.zeros = torch.empty((n, sz["zeros"] // n), dtype=torch.uint8, device=dev)
        if sz["absmax"]:
            qw.absmax = torch.empty(sz["absmax"] // 4, dtype=torch.float32, device=dev)
        if sz["absmax_q"]:
            qw.absmax_q = torch.empty(sz["absmax_q"], dtype=torch.int8, device=dev)
            qw.absmax_scale = torch.empty(sz["absmax_scale"] // 4, dtype=torch.float32, device=dev)
        return qw


def lbq_quantize(W: torch.Tensor, fmt: str = "minmax", bits: int = 4, group: Optional[int] = None,
                 double_quant: bool = True, out: Optional[QuantizedWeight] = None, compact: bool = False,
                 dq_offset: bool = False) -> QuantizedWeight:
    """Quantize a device fp32 weight W[n][k] (see ``lbq_quantize`` in lbq.h)."""
    if W.dim() != 2:
        raise ValueError("W must be 2-D [n, k]")
    _need(W, "W", torch.float32)
    desc = make_desc(fmt, W.shape[0], W.shape[1], bits, group, double_quant, compact, dq_offset)
    qw = out if out is not None else QuantizedWeight.empty(desc, W.device)
    q = qw.qtensor()
    check(lib.lbq_quantize(ctypes.byref(desc), W.data_ptr(), ctypes.byref(q), _stream(W.device)),
          "lbq_quantize")
    qw.desc = desc
    return qw


def lbq_dequant(qw: QuantizedWeight, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """bf16 W_hat[n][k] (see ``lbq_dequant`` in lbq.h)."""
    if out is None:
        out = torch.empty((qw.n, qw.k), dtype=torch.bfloat16, device=qw.device)
    _need(out, "out", torch.bfloat16, (qw.n, qw.k))
    q = qw.qtensor()
    check(lib.lbq_dequant(ctypes.byref(qw.desc), ctypes.byref(q), out.data_ptr(), _stream(qw.device)),
          "lbq_dequant")
    return out


def lbq_linear_workspace_bytes(qw: QuantizedWeight, m: int) -> int:
    return lib.lbq_linear_workspace_bytes(ctypes.byref(qw.desc), m)


def lbq_lora_workspace_bytes(qw: QuantizedWeight, m: int, r: int) -> int:
    return lib.lbq_lora_workspace_bytes(ctypes.byref(qw.desc), m, r)


def _ws(nbytes: int, device) -> Optional[torch.Tensor]:
    if nbytes == 0:
        return None
    return torch.empty(((nbytes + 15) // 16) * 16, dtype=torch.uint8, device=device)


def lbq_linear_fwd(X: torch.Tensor, qw: QuantizedWeight, out: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Y = X . deq(W)^T in bf16 (see ``lbq_linear_fwd`` in lbq.h).  With
    ``qw.out_rows`` set, ``out`` must be given and only those columns are written."""
    _need(X, "X", torch.bfloat16)
    m = X.shape[0]
    if X.dim() != 2 or X.shape[1] != qw.k:
        raise ValueError(f"X must be [m, {qw.k}]")
    if out is None:
        if qw.out_rows is not None:
            raise ValueError("out must be given when out_rows is set")
        out = torch.empty((m, qw.n), dtype=torch.bfloat16, device=X.device)
    if out.dtype != torch.bfloat16 or out.dim() != 2 or out.shape[0] != m or out.stride(1) != 1:
        raise ValueError("out must be bf16 [m, >=n] with unit column stride")
    nbytes = lbq_linear_workspace_bytes(qw, m)
    if workspace is None:
        workspace = _ws(nbytes, X.device)
    q = qw.qtensor()
    check(lib.lbq_linear_fwd(ctypes.byref(qw.desc), ctypes.byref(q), X.data_ptr(), m, out.data_ptr(),
                             out.stride(0), _ptr(workspace), 0 if workspace is None else workspace.numel(),
                             _stream(X.device)), "lbq_linear_fwd")
    return out


def lbq_linear_fwd_noalloc(X: torch.Tensor, qw: QuantizedWeight, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """``lbq_linear_fwd`` without a workspace (see ``lbq_linear_fwd_noalloc`` in
    lbq.h): the library's own per-device scratch array holds the partial sums."""
    _need(X, "X", torch.bfloat16)
    m = X.shape[0]
    if X.dim() != 2 or X.shape[1] != qw.k:
        raise ValueError(f"X must be [m, {qw.k}]")
    if out is None:
        if qw.out_rows is not None:
            raise ValueError("out must be given when out_rows is set")
        out = torch.empty((m, qw.n), dtype=torch.bfloat16, device=X.device)
    if out.dtype != torch.bfloat16 or out.dim() != 2 or out.shape[0] != m or out.stride(1) != 1:
        raise ValueError("out must be bf16 [m, >=n] with unit column stride")
    q = qw.qtensor()
    check(lib.lbq_linear_fwd_noalloc(ctypes.byref(qw.desc), ctypes.byref(q), X.data_ptr(), m, out.data_ptr(),
                                     out.stride(0), _stream(X.device)), "lbq_linear_fwd_noalloc")
    return out


def lbq_linear_fwd_grouped_workspace_bytes(qws, m: int) -> int:
    descs = (Desc * len(qws))(*[q.desc for q in qws])
    return lib.lbq_linear_fwd_grouped_workspace_bytes(len(qws), descs, m)


def lbq_linear_fwd_grouped(X: torch.Tensor, qws, outs=None, workspace: Optional[torch.Tensor] = None):
    """Ys[i] = X . deq(W_i)^T for weights that share X and k (see
    ``lbq_linear_fwd_grouped`` in lbq.h).  Returns the list of outputs; an
    ``outs`` entry is required where that weight has ``out_rows`` (several
    weights may scatter into one tensor)."""
    _need(X, "X", torch.bfloat16)
    qws = list(qws)
    count = len(qws)
    if not 1 <= count <= LBQ_MAX_GROUP:
        raise ValueError(f"between 1 and {LBQ_MAX_GROUP} weights")
    m = X.shape[0]
    if X.dim() != 2 or any(q.k != X.shape[1] for q in qws):
        raise ValueError("X must be [m, k] with every weight's k")
    outs = list(outs) if outs is not None else [None] * count
    if len(outs) != count:
        raise ValueError("one output per weight")
    for i, (q, o) in enumerate(zip(qws, outs)):
        if o is None:
            if q.out_rows is not None:
                raise ValueError(f"outs[{i}] must be given when out_rows is set")
            outs[i] = torch.empty((m, q.n), dtype=torch.bfloat16, device=X.device)
        o = outs[i]
        if o.dtype != torch.bfloat16 or o.dim() != 2 or o.shape[0] != m or o.stride(1) != 1:
            raise ValueError(f"outs[{i}] must be bf16 [m, >=n] with unit column stride")
    descs = (Desc * count)(*[q.desc for q in qws])
    qts = (QTensor * count)(*[q.qtensor() for q in qws])
    ys = (ctypes.c_void_p * count)(*[o.data_ptr() for o in outs])
    ldys = (ctypes.c_int64 * count)(*[o.stride(0) for o in outs])
    nbytes = lib.lbq_linear_fwd_grouped_workspace_bytes(count, descs, m)
    if workspace is None:
        workspace = _ws(nbytes, X.device)
    check(lib.lbq_linear_fwd_grouped(count, descs, qts, X.data_ptr(), m, ys, ldys, _ptr(workspace),
                                     0 if workspace is None else workspace.numel(), _stream(X.device)),
          "lbq_linear_fwd_grouped")
    return outs


def lbq_linear_bwd_dx(dY: torch.Tensor, qw: QuantizedWeight,
                      out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """dX = dY . deq(W) in bf16 (see ``lbq_linear_bwd_dx`` in lbq.h)."""
    _need(dY, "dY", torch.bfloat16)
    if dY.dim() != 2 or dY.shape[1] != qw.n:
        raise ValueError(f"dY must be [m, {qw.n}]")
    m = dY.shape[0]
    if out is None:
        out = torch.empty((m, qw.k), dtype=torch.bfloat16, device=dY.device)
    _need(out, "out", torch.bfloat16, (m, qw.k))
    q = qw.qtensor()
    check(lib.lbq_linear_bwd_dx(ctypes.byref(qw.desc), ctypes.byref(q), dY.data_ptr(), m,
                                out.data_ptr(), _stream(dY.device)), "lbq_linear_bwd_dx")
    return out


def lbq_linear_bwd_dx_grouped(dYs, qws, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """dX = sum_i dYs[i] . deq(W_i) in bf16 for weights of one format that
    share X and k (see ``lbq_linear_bwd_dx_grouped`` in lbq.h)."""
    qws, dYs = list(qws), list(dYs)
    count = len(qws)
    if not 1 <= count <= LBQ_MAX_GROUP or len(dYs) != count:
        raise ValueError(f"between 1 and {LBQ_MAX_GROUP} weights, one dY each")
    for i, (d, q) in enumerate(zip(dYs, qws)):
        _need(d, f"dYs[{i}]", torch.bfloat16)
        if d.dim() != 2 or d.shape[1] != q.n or d.shape[0] != dYs[0].shape[0]:
            raise ValueError(f"dYs[{i}] must be [m, {q.n}]")
        if q.k != qws[0].k:
            raise ValueError("every weight must have the same k")
    m, k = dYs[0].shape[0], qws[0].k
    if out is None:
        out = torch.empty((m, k), dtype=torch.bfloat16, device=dYs[0].device)
    _need(out, "out", torch.bfloat16, (m, k))
    descs = (Desc * count)(*[q.desc for q in qws])
    qts = (QTensor * count)(*[q.qtensor() for q in qws])
    dps = (ctypes.c_void_p * count)(*[d.data_ptr() for d in dYs])
    check(lib.lbq_linear_bwd_dx_grouped(count, descs, qts, dps, m, out.data_ptr(), _stream(dYs[0].device)),
          "lbq_linear_bwd_dx_grouped")
    return out


def lbq_lora_fwd(X: torch.Tensor, qw: QuantizedWeight, A: torch.Tensor, B: torch.Tensor,
                 sigma: float, out: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Y = X . deq(W)^T + sigma (X A^T) B^T (see ``lbq_lora_fwd`` in lbq.h)."""
    _need(X, "X", torch.bfloat16)
    _need(A, "A", torch.bfloat16)
    _need(B, "B", torch.bfloat16)
    m = X.shape[0]
    r = A.shape[0]
    if A.shape[1] != qw.k or B.shape != (qw.n, r):
        raise ValueError("A must be [r, k] and B [n, r]")
    if out is None:
        if qw.out_rows is not None:
            raise ValueError("out must be given when out_rows is set")
        out = torch.empty((m, qw.n), dtype=torch.bfloat16, device=X.device)
    nbytes = lbq_lora_workspace_bytes(qw, m, r)
    if workspace is None:
        workspace = _ws(nbytes, X.device)
    q = qw.qtensor()
    check(lib.lbq_lora_fwd(ctypes.byref(qw.desc), ctypes.byref(q), X.data_ptr(), m, A.data_ptr(),
                           B.data_ptr(), r, float(sigma), out.data_ptr(), out.stride(0),
                           _ptr(workspace), 0 if workspace is None else workspace.numel(),
                           _stream(X.device)), "lbq_lora_fwd")
    return out


def lbq_lora_bwd_workspace_bytes(qw: QuantizedWeight, m: int, r: int) -> int:
    return lib.lbq_lora_bwd_workspace_bytes(ctypes.byref(qw.desc), m, r)


def lbq_lora_bwd(X: torch.Tensor, dY: torch.Tensor, qw: QuantizedWeight, A: torch.Tensor,
                 B: torch.Tensor, sigma: float, dX: Optional[torch.Tensor] = None,
                 dA: Optional[torch.Tensor] = None, dB: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None):
    """(dX bf16 [m, k], dA fp32 [r, k], dB fp32 [n, r]) of ``lbq_lora_fwd`` for a
    frozen weight (see ``lbq_lora_bwd`` in lbq.h)."""
    _need(X, "X", torch.bfloat16)
    _need(dY, "dY", torch.bfloat16)
    _need(A, "A", torch.bfloat16)
    _need(B, "B", torch.bfloat16)
    m, r = X.shape[0], A.shape[0]
    if X.dim() != 2 or X.shape[1] != qw.k or dY.shape != (m, qw.n):
        raise ValueError(f"X must be [m, {qw.k}] and dY [m, {qw.n}]")
    if A.shape[1] != qw.k or B.shape != (qw.n, r):
        raise ValueError("A must be [r, k] and B [n, r]")
    dev = X.device
    if dX is None:
        dX = torch.empty((m, qw.k), dtype=torch.bfloat16, device=dev)
    if dA is None:
        dA = torch.empty((r, qw.k), dtype=torch.float32, device=dev)
    if dB is None:
        dB = torch.empty((qw.n, r), dtype=torch.float32, device=dev)
    _need(dX, "dX", torch.bfloat16, (m, qw.k))
    _need(dA, "dA", torch.float32, (r, qw.k))
    _need(dB, "dB", torch.float32, (qw.n, r))
    nbytes = lbq_lora_bwd_workspace_bytes(qw, m, r)
    if workspace is None:
        workspace = _ws(nbytes, dev)
    q = qw.qtensor()
    check(lib.lbq_lora_bwd(ctypes.byref(qw.desc), ctypes.byref(q), X.data_ptr(), dY.data_ptr(), m,
                           A.data_ptr(), B.data_ptr(), r, float(sigma), dX.data_ptr(), dA.data_ptr(),
                           dB.data_ptr(), _ptr(workspace), 0 if workspace is None else workspace.numel(),
                           _stream(dev)), "lbq_lora_bwd")
    return dX, dA, dB


class _LoraLinearFn(torch.autograd.Function):
    """Y = X . deq(W)^T + sigma (X . A^T) . B^T with a frozen quantized W:
    forward through ``lbq_lora_fwd``, backward through ``lbq_lora_bwd`` (the
    gradient reaches X and the adapters, never W)."""

    @staticmethod
    def forward(ctx, X, A, B, qw, sigma):
        lead = X.shape[:-1]
        X2 = X.reshape(-1, qw.k).to(torch.bfloat16).contiguous()
        A16 = A.detach().to(torch.bfloat16).contiguous()
        B16 = B.detach().to(torch.bfloat16).contiguous()
        Y = lbq_lora_fwd(X2, qw, A16, B16, sigma)
        ctx.save_for_backward(X2, A16, B16)
        ctx.qw, ctx.sigma, ctx.x_shape, ctx.x_dtype = qw, sigma, X.shape, X.dtype
        ctx.a_dtype, ctx.b_dtype = A.dtype, B.dtype
        return Y.reshape(*lead, qw.n)

    @staticmethod
    def backward(ctx, dY):
        X2, A16, B16 = ctx.saved_tensors
        dY2 = dY.reshape(-1, ctx.qw.n).to(torch.bfloat16).contiguous()
        dX, dA, dB = lbq_lora_bwd(X2, dY2, ctx.qw, A16, B16, ctx.sigma)
        return (dX.reshape(ctx.x_shape).to(ctx.x_dtype), dA.to(ctx.a_dtype), dB.to(ctx.b_dtype), None, None)


class LbqLoraLinear(torch.nn.Module):
    """A frozen low-bit linear layer with trainable LoRA adapters (r <= 64,
    n % 64 == 0).  A [r, k] and B [n, r] are parameters (fp32 masters by
    default; the kernels see them rounded to bf16); B starts at zero, so the
    adapted layer starts equal to the frozen one."""

    def __init__(self, qw: QuantizedWeight, r: int = 16, lora_alpha: float = 16.0,
                 dtype: torch.dtype = torch.float32, generator: Optional[torch.Generator] = None):
        super().__init__()
        if not 1 <= r <= 64 or qw.n % 64 != 0:
            raise ValueError("LbqLoraLinear needs 1 <= r <= 64 and n % 64 == 0")
        self.qw = qw
        self.sigma = lora_alpha / r
        bound = 1.0 / qw.k ** 0.5
        a = torch.empty((r, qw.k), dtype=dtype, device=qw.device)
        a.uniform_(-bound, bound, generator=generator)
        self.A = torch.nn.Parameter(a)
        self.B = torch.nn.Parameter(torch.zeros((qw.n, r), dtype=dtype, device=qw.device))

    def forward(self, X: torch.Tensor) -> torch.Tensor:
        return _LoraLinearFn.apply(X, self.A, self.B, self.qw, self.sigma)
