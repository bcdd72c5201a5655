"""Weight-only quantized GEMM (fpA_intB: W4A16 groupwise, W8A16 per channel,
top-k MoE) for AMD MI355X (gfx950).

Thin torch-facing wrappers over the C ABI in ``include/qgemm.h``: they check
tensor placement, flatten leading dimensions, pass raw device pointers and
torch's current HIP stream, and raise ``QGemmError`` on any non-OK status.
Every computation runs in the library's HIP kernels; there is no other path.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from ._abi import (QG_BF16, QG_FP16, QG_FP32, QG_LAYOUT_PORTABLE, QG_LAYOUT_TILED,
                   QG_MOE_NORM_NONE, QG_MOE_RENORMALIZE, QG_NONE, QG_W8A8_PER_CHANNEL,
                   QG_W8A8_PER_TOKEN, QGemmError, check, lib)

__all__ = [
    "QGemmError", "lib", "repack_w4", "unrepack_w4", "repack_w8", "unrepack_w8", "repack_w8_kn",
    "unrepack_w8_kn", "quantize_w4", "dequant_w4", "dequant_w8", "gemm_w4a16", "gemm_w8a16",
    "moe_grouped", "moe_workspace_size", "gemm_workspace_size", "dtype_code", "gemm_w8a8",
    "w8a8_workspace_size", "embed_w4", "embed_w8", "read_probe", "lds_probe", "set_override", "clear_override",
    "moe_grouped_noalloc",
]

_CODES = {torch.bfloat16: QG_BF16, torch.float16: QG_FP16, torch.float32: QG_FP32}


def dtype_code(dt: Optional[torch.dtype]) -> int:
    if dt is None:
        return QG_NONE
    if dt not in _CODES:
        raise QGemmError("dtype", 4, f"unsupported dtype {dt}")
    return _CODES[dt]


def _dev(t: torch.Tensor, name: str) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise QGemmError(name, 1, f"{name} must be a device tensor (got {t.device})")
    if not t.is_contiguous():
        raise QGemmError(name, 2, f"{name} must be contiguous")
    return t


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(t: torch.Tensor):
    """Raw handle of torch's current stream on t's device (a hipStream_t)."""
    if _raw_stream is not None:
        return _raw_stream(t.get_device())
    return torch.cuda.current_stream(t.device).cuda_stream


# -- operand checks: shapes and dtypes, before any pointer reaches the library --
# The C ABI takes raw pointers and sizes, so a tensor of the wrong shape or
# dtype would be read past its end or misread; these raise instead.

_SHAPE, _DTYPE = 2, 4
_ACT = (torch.bfloat16, torch.float16)


def _need(cond: bool, func: str, status: int, msg: str) -> None:
    if not cond:
        raise QGemmError(func, status, msg)


def _shape(t) -> tuple:
    return tuple(t.shape)


def _check_groups(func: str, name: str, t: torch.Tensor, dtype, rows: int, k: int, group: int,
                  lead: tuple = ()) -> None:
    """scales / zeros: `dtype`, shape lead + [rows, k / group] (groupwise) or
    lead + [rows] (group -1 or k: one per row; a trailing 1 is accepted)."""
    _need(t.dtype == dtype, func, _DTYPE, f"{name} must be {dtype} (got {t.dtype})")
    if group in (-1, k):
        ok = _shape(t) in (lead + (rows,), lead + (rows, 1))
        want = f"{list(lead + (rows,))}"
    elif group > 0 and k % group == 0:
        ok = _shape(t) == lead + (rows, k // group)
        want = f"{list(lead + (rows, k // group))}"
    else:
        return   # the library rejects the group size itself
    _need(ok, func, _SHAPE, f"{name} must be {want} (got {list(t.shape)})")


def _check_out(func: str, out: torch.Tensor, dtype, m: int, n: int) -> None:
    _need(out.dtype == dtype, func, _DTYPE, f"out must be {dtype} (got {out.dtype})")
    _need(out.dim() >= 1 and out.shape[-1] == n and out.numel() == m * n, func, _SHAPE,
          f"out must hold [{m}, {n}] (got {list(out.shape)})")


def _check_bias(func: str, bias: Optional[torch.Tensor], n: int) -> None:
    if bias is None:
        return
    _need(bias.dtype in _ACT, func, _DTYPE, f"bias must be bf16 or fp16 (got {bias.dtype})")
    _need(_shape(bias) == (n,), func, _SHAPE, f"bias must be [{n}] (got {list(bias.shape)})")


# -- dispatch override (tests and tuning) -------------------------------------

_override: dict = {}


def set_override(**choices) -> None:
    """Force dispatch choices for later calls (qg_set_override): path,
    prefill_tile, splitk, moe_tile, w8a8_tile, w8a8_split.  Merges with the
    choices set before; a value of None returns that key to automatic."""
    for key, val in choices.items():
        if val is None:
            _override.pop(key, None)
        else:
            _override[key] = val
    spec = ",".join(f"{k}={v}" for k, v in _override.items())
    check("qg_set_override", lib().qg_set_override(spec.encode()))


def clear_override() -> None:
    """Every dispatch choice automatic again."""
    _override.clear()
    check("qg_set_override", lib().qg_set_override(None))


# -- load-side repack -------------------------------------------------------

def repack_w4(packed: torch.Tensor) -> torch.Tensor:
    """Portable int4 [n, k/2] uint8 -> tiled layout (same shape and bytes)."""
    _need(packed.dtype == torch.uint8 and packed.dim() == 2, "qrepack_w4", _DTYPE,
          "packed must be a 2-D uint8 tensor [n, k/2]")
    _dev(packed, "packed")
    n, half = packed.shape
    out = torch.empty_like(packed)
    check("qrepack_w4", lib().qrepack_w4(_ptr(packed), _ptr(out), n, 2 * half, _stream(packed)))
    return out


def unrepack_w4(tiled: torch.Tensor) -> torch.Tensor:
    _need(tiled.dtype == torch.uint8 and tiled.dim() == 2, "qunrepack_w4", _DTYPE,
          "tiled must be a 2-D uint8 tensor [n, k/2]")
    _dev(tiled, "tiled")
    n, half = tiled.shape
    out = torch.empty_like(tiled)
    check("qunrepack_w4", lib().qunrepack_w4(_ptr(tiled), _ptr(out), n, 2 * half, _stream(tiled)))
    return out


def repack_w8(codes: torch.Tensor) -> torch.Tensor:
    """Portable int8 [n, k] -> tiled layout (same shape, offset-binary bytes)."""
    _need(codes.dtype == torch.int8 and codes.dim() == 2, "qrepack_w8", _DTYPE,
          "codes must be a 2-D int8 tensor [n, k]")
    _dev(codes, "codes")
    n, k = codes.shape
    out = torch.empty_like(codes)
    check("qrepack_w8", lib().qrepack_w8(_ptr(codes), _ptr(out), n, k, _stream(codes)))
    return out


def unrepack_w8(tiled: torch.Tensor) -> torch.Tensor:
    _need(tiled.dtype == torch.int8 and tiled.dim() == 2, "qunrepack_w8", _DTYPE,
          "tiled must be a 2-D int8 tensor [n, k]")
    _dev(tiled, "tiled")
    n, k = tiled.shape
    out = torch.empty_like(tiled)
    check("qunrepack_w8", lib().qunrepack_w8(_ptr(tiled), _ptr(out), n, k, _stream(tiled)))
    return out


def repack_w8_kn(codes_kn: torch.Tensor) -> torch.Tensor:
    """int8 [k, n] (K-major) -> tiled layout [n, k] (as repack_w8 of the transpose)."""
    _need(codes_kn.dtype == torch.int8 and codes_kn.dim() == 2, "qrepack_w8_kn", _DTYPE,
          "codes_kn must be a 2-D int8 tensor [k, n]")
    _dev(codes_kn, "codes_kn")
    k, n = codes_kn.shape
    out = torch.empty((n, k), dtype=codes_kn.dtype, device=codes_kn.device)
    check("qrepack_w8_kn", lib().qrepack_w8_kn(_ptr(codes_kn), _ptr(out), n, k, _stream(codes_kn)))
    return out


def unrepack_w8_kn(tiled: torch.Tensor) -> torch.Tensor:
    """Tiled int8 [n, k] -> int8 [k, n] (K-major)."""
    _need(tiled.dtype == torch.int8 and tiled.dim() == 2, "qunrepack_w8_kn", _DTYPE,
          "tiled must be a 2-D int8 tensor [n, k]")
    _dev(tiled, "tiled")
    n, k = tiled.shape
    out = torch.empty((k, n), dtype=tiled.dtype, device=tiled.device)
    check("qunrepack_w8_kn", lib().qunrepack_w8_kn(_ptr(tiled), _ptr(out), n, k, _stream(tiled)))
    return out


# -- quantizer -----------------------------------------------------------------

def quantize_w4(W: torch.Tensor, group_size: int = 64, sz_dtype: Optional[torch.dtype] = None):
    """Groupwise min/max int4 quantization of W [n, k] (bf16, fp16 or fp32).

    Returns (packed uint8 [n, k/2] in the portable layout, scales, zeros
    [n, k/group] in sz_dtype, default W's dtype).
    """
    _need(W.dtype in _ACT + (torch.float32,) and W.dim() == 2, "qquantize_w4", _DTYPE,
          "W must be a 2-D bf16, fp16 or fp32 tensor [n, k]")
    sz_dtype = W.dtype if sz_dtype is None else sz_dtype
    _need(sz_dtype in _ACT + (torch.float32,), "qquantize_w4", _DTYPE,
          "sz_dtype must be bf16, fp16 or fp32")
    _dev(W, "W")
    n, k = W.shape
    packed = torch.empty((n, k // 2), dtype=torch.uint8, device=W.device)
    ng = k // group_size if group_size > 0 else 0
    scales = torch.empty((n, ng), dtype=sz_dtype, device=W.device)
    zeros = torch.empty((n, ng), dtype=sz_dtype, device=W.device)
    check("qquantize_w4", lib().qquantize_w4(_ptr(W), _ptr(packed), _ptr(scales), _ptr(zeros), n, k,
                                             group_size, dtype_code(W.dtype), dtype_code(sz_dtype),
                                             _stream(W)))
    return packed, scales, zeros


# -- dequant hook ------------------------------------------------------------

def dequant_w4(tiled: torch.Tensor, scales: torch.Tensor, zeros: Optional[torch.Tensor],
               group_size: int, out_dtype: torch.dtype = torch.float32) -> torch.Tensor:
    """Tiled int4 -> W [n, k]; zeros None = scale-only, group_size -1 = per channel."""
    f = "qdequant_w4"
    _need(tiled.dtype == torch.uint8 and tiled.dim() == 2, f, _DTYPE,
          "tiled must be a 2-D uint8 tensor [n, k/2]")
    _need(scales.dtype in _ACT, f, _DTYPE, "scales must be bf16 or fp16")
    _check_groups(f, "scales", scales, scales.dtype, tiled.shape[0], 2 * tiled.shape[1], group_size)
    if zeros is not None:
        _check_groups(f, "zeros", zeros, scales.dtype, tiled.shape[0], 2 * tiled.shape[1], group_size)
    _need(out_dtype in (torch.float32, scales.dtype), f, _DTYPE,
          "out_dtype must be fp32 or the scales' dtype")
    for t, nm in ((tiled, "tiled"), (scales, "scales"), (zeros, "zeros")):
        if t is not None:
            _dev(t, nm)
    n, half = tiled.shape
    out = torch.empty((n, 2 * half), dtype=out_dtype, device=tiled.device)
    check("qdequant_w4", lib().qdequant_w4(_ptr(tiled), _ptr(scales), _ptr(zeros), _ptr(out), n,
                                           2 * half, group_size, dtype_code(scales.dtype),
                                           dtype_code(out_dtype), _stream(tiled)))
    return out


def dequant_w8(tiled: torch.Tensor, scales: torch.Tensor,
               out_dtype: torch.dtype = torch.float32, group_size: int = -1) -> torch.Tensor:
    f = "qdequant_w8"
    _need(tiled.dtype == torch.int8 and tiled.dim() == 2, f, _DTYPE,
          "tiled must be a 2-D int8 tensor [n, k]")
    _need(scales.dtype in _ACT, f, _DTYPE, "scales must be bf16 or fp16")
    _check_groups(f, "scales", scales, scales.dtype, tiled.shape[0], tiled.shape[1], group_size)
    _need(out_dtype in (torch.float32, scales.dtype), f, _DTYPE,
          "out_dtype must be fp32 or the scales' dtype")
    _dev(tiled, "tiled")
    _dev(scales, "scales")
    n, k = tiled.shape
    out = torch.empty((n, k), dtype=out_dtype, device=tiled.device)
    check("qdequant_w8", lib().qdequant_w8(_ptr(tiled), _ptr(scales), _ptr(out), n, k, group_size,
                                           dtype_code(scales.dtype), dtype_code(out_dtype),
                                           _stream(tiled)))
    return out


# -- GEMM --------------------------------------------------------------------

def gemm_workspace_size(m: int, n: int, k: int, group_size: int, weight_bits: int) -> int:
    return int(lib().qgemm_workspace_size(m, n, k, group_size, weight_bits))


def _workspace(m: int, n: int, k: int, group_size: int, bits: int, device,
               given: Optional[torch.Tensor]):
    """(tensor, bytes) of workspace for a GEMM: the caller's, else a fresh
    one when the library asks for any (split-K partials), else (None, 0)."""
    if given is not None:
        _dev(given, "workspace")
        return given, given.numel() * given.element_size()
    need = int(lib().qgemm_workspace_size(m, n, k, group_size, bits))
    if need == 0:
        return None, 0
    return torch.empty(need, dtype=torch.uint8, device=device), need


def gemm_w4a16(A: torch.Tensor, B_tiled: torch.Tensor, scales: torch.Tensor,
               zeros: Optional[torch.Tensor], bias: Optional[torch.Tensor] = None,
               group_size: int = 64, out: Optional[torch.Tensor] = None,
               workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """C = A . dequant(B)^T (+ bias); A [..., k] bf16/fp16, B tiled int4.

    group_size 64 / 128 (scales [n, k/g]) or -1 (one per channel, [n]);
    zeros None for scale-only weights, w = (q - 8) * s.
    """
    f = "qgemm_w4a16"
    _need(A.dtype in _ACT and A.dim() >= 1, f, _DTYPE, f"A must be bf16 or fp16 (got {A.dtype})")
    k = A.shape[-1]
    m = A.numel() // k if k else 0
    _need(B_tiled.dtype == torch.uint8 and B_tiled.dim() == 2, f, _DTYPE,
          "B_tiled must be a 2-D uint8 tensor [n, k/2]")
    _need(2 * B_tiled.shape[1] == k, f, _SHAPE,
          f"B_tiled must be [n, {k // 2}] for k = {k} (got {list(B_tiled.shape)})")
    n = B_tiled.shape[0]
    _check_groups(f, "scales", scales, A.dtype, n, k, group_size)
    if zeros is not None:
        _check_groups(f, "zeros", zeros, A.dtype, n, k, group_size)
    _check_bias(f, bias, n)
    if out is not None:
        _check_out(f, out, A.dtype, m, n)
    _dev(A, "A")
    for t, nm in ((B_tiled, "B_tiled"), (scales, "scales"), (zeros, "zeros")):
        if t is not None:
            _dev(t, nm)
    if bias is not None:
        _dev(bias, "bias")
    lead = A.shape[:-1]
    A2 = A.reshape(-1, k)
    C = out if out is not None else torch.empty((m, n), dtype=A.dtype, device=A.device)
    _dev(C, "out")
    ws, ws_bytes = _workspace(m, n, k, group_size, 4, A.device, workspace)
    check("qgemm_w4a16", lib().qgemm_w4a16(
        _ptr(A2), _ptr(B_tiled), _ptr(scales), _ptr(zeros), _ptr(bias), _ptr(C), m, n, k,
        group_size, dtype_code(A.dtype), dtype_code(None if bias is None else bias.dtype),
        _ptr(ws), ws_bytes, _stream(A)))
    return C.reshape(*lead, n)


def gemm_w8a16(A: torch.Tensor, B_tiled: torch.Tensor, scales: torch.Tensor,
               bias: Optional[torch.Tensor] = None, group_size: int = -1,
               out: Optional[torch.Tensor] = None,
               workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """C = A . dequant(B)^T (+ bias); A [..., k] bf16/fp16, B tiled int8."""
    f = "qgemm_w8a16"
    _need(A.dtype in _ACT and A.dim() >= 1, f, _DTYPE, f"A must be bf16 or fp16 (got {A.dtype})")
    k = A.shape[-1]
    m = A.numel() // k if k else 0
    _need(B_tiled.dtype == torch.int8 and B_tiled.dim() == 2, f, _DTYPE,
          "B_tiled must be a 2-D int8 tensor [n, k]")
    _need(B_tiled.shape[1] == k, f, _SHAPE,
          f"B_tiled must be [n, {k}] (got {list(B_tiled.shape)})")
    n = B_tiled.shape[0]
    _check_groups(f, "scales", scales, A.dtype, n, k, group_size)
    _check_bias(f, bias, n)
    if out is not None:
        _check_out(f, out, A.dtype, m, n)
    _dev(A, "A")
    _dev(B_tiled, "B_tiled")
    _dev(scales, "scales")
    if bias is not None:
        _dev(bias, "bias")
    lead = A.shape[:-1]
    A2 = A.reshape(-1, k)
    C = out if out is not None else torch.empty((m, n), dtype=A.dtype, device=A.device)
    _dev(C, "out")
    ws, ws_bytes = _workspace(m, n, k, group_size, 8, A.device, workspace)
    check("qgemm_w8a16", lib().qgemm_w8a16(
        _ptr(A2), _ptr(B_tiled), _ptr(scales), _ptr(bias), _ptr(C), m, n, k, group_size,
        dtype_code(A.dtype), dtype_code(None if bias is None else bias.dtype), _ptr(ws),
        ws_bytes, _stream(A)))
    return C.reshape(*lead, n)


# -- W8A8 ----------------------------------------------------------------------

def w8a8_workspace_size(m: int, n: int, k: int) -> int:
    return int(lib().qgemm_w8a8_workspace_size(m, n, k))


def gemm_w8a8(A: torch.Tensor, B: torch.Tensor, alpha_row: torch.Tensor,
              alpha_col: torch.Tensor, out_dtype: torch.dtype = torch.float16,
              out: Optional[torch.Tensor] = None,
              workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """C = (A_int8 . B_int8^T) * alpha_row * alpha_col; A [..., k] int8,
    B [n, k] int8, alpha_row fp32 [m] (per token) or [1], alpha_col fp32 [n]
    (per channel) or [1]; the quant mode follows the scale lengths."""
    f = "qgemm_w8a8"
    _need(A.dtype == torch.int8 and A.dim() >= 1, f, _DTYPE, "A must be int8")
    _need(B.dtype == torch.int8 and B.dim() == 2, f, _DTYPE, "B must be a 2-D int8 tensor [n, k]")
    _need(alpha_row.dtype == torch.float32 and alpha_col.dtype == torch.float32, f, _DTYPE,
          "alpha_row and alpha_col must be fp32")
    k = A.shape[-1]
    _need(B.shape[1] == k, f, _SHAPE, f"B must be [n, {k}] (got {list(B.shape)})")
    _dev(A, "A")
    _dev(B, "B")
    _dev(alpha_row, "alpha_row")
    _dev(alpha_col, "alpha_col")
    lead = A.shape[:-1]
    A2 = A.reshape(-1, k)
    m, n = A2.shape[0], B.shape[0]
    if alpha_row.numel() not in (1, m) or alpha_col.numel() not in (1, n):
        raise QGemmError("qgemm_w8a8", 2, "alpha_row must hold 1 or m values, alpha_col 1 or n")
    mode = ((QG_W8A8_PER_TOKEN if alpha_row.numel() == m and m > 1 else 0)
            | (QG_W8A8_PER_CHANNEL if alpha_col.numel() == n and n > 1 else 0))
    C = out if out is not None else torch.empty((m, n), dtype=out_dtype, device=A.device)
    _dev(C, "out")
    if tuple(C.shape) != (m, n):
        raise QGemmError("qgemm_w8a8", 2, f"out must be [{m}, {n}]")
    need = w8a8_workspace_size(m, n, k)
    ws = workspace
    if ws is None and need:
        ws = torch.empty(need, dtype=torch.uint8, device=A.device)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    check("qgemm_w8a8", lib().qgemm_w8a8(
        _ptr(A2), _ptr(B), mode, _ptr(alpha_col), _ptr(alpha_row), _ptr(C), m, n, k,
        dtype_code(C.dtype), _ptr(ws), ws_bytes, _stream(A)))
    return C.reshape(*lead, n)


# -- embedding lookup ----------------------------------------------------------

def _embed_out(ids, hidden, act_dtype, out_dtype, device):
    return torch.empty((*ids.shape, hidden), dtype=out_dtype or act_dtype, device=device)


def embed_w4(ids: torch.Tensor, table: torch.Tensor, scales: torch.Tensor,
             zeros: Optional[torch.Tensor], group_size: int, tiled: bool = True,
             out_dtype: Optional[torch.dtype] = None) -> torch.Tensor:
    """Rows ids of the int4 table, dequantized: [*ids.shape, hidden].  The
    table is the tiled [vocab, hidden/2] GEMM weight (tiled=True) or the
    portable one; scales (and zeros) set the activation dtype."""
    f = "qembed_w4"
    _need(ids.dtype == torch.int32, f, _DTYPE, "ids must be int32")
    _need(table.dtype == torch.uint8 and table.dim() == 2, f, _DTYPE,
          "table must be a 2-D uint8 tensor [vocab, hidden/2]")
    _need(scales.dtype in _ACT, f, _DTYPE, "scales must be bf16 or fp16")
    _check_groups(f, "scales", scales, scales.dtype, table.shape[0], 2 * table.shape[1], group_size)
    if zeros is not None:
        _check_groups(f, "zeros", zeros, scales.dtype, table.shape[0], 2 * table.shape[1], group_size)
    for t, name in ((ids, "ids"), (table, "table"), (scales, "scales")):
        _dev(t, name)
    if zeros is not None:
        _dev(zeros, "zeros")
    vocab, hidden = table.shape[0], table.shape[1] * 2
    out = _embed_out(ids, hidden, scales.dtype, out_dtype, table.device)
    check("qembed_w4", lib().qembed_w4(
        _ptr(ids), ids.numel(), _ptr(table), QG_LAYOUT_TILED if tiled else QG_LAYOUT_PORTABLE,
        _ptr(scales), _ptr(zeros), _ptr(out), vocab, hidden, group_size, dtype_code(scales.dtype),
        dtype_code(out.dtype), _stream(table)))
    return out


def embed_w8(ids: torch.Tensor, table: torch.Tensor, scales: torch.Tensor, group_size: int = -1,
             tiled: bool = True, out_dtype: Optional[torch.dtype] = None) -> torch.Tensor:
    """Rows ids of the int8 table [vocab, hidden], dequantized."""
    f = "qembed_w8"
    _need(ids.dtype == torch.int32, f, _DTYPE, "ids must be int32")
    _need(table.dtype == torch.int8 and table.dim() == 2, f, _DTYPE,
          "table must be a 2-D int8 tensor [vocab, hidden]")
    _need(scales.dtype in _ACT, f, _DTYPE, "scales must be bf16 or fp16")
    _check_groups(f, "scales", scales, scales.dtype, table.shape[0], table.shape[1], group_size)
    for t, name in ((ids, "ids"), (table, "table"), (scales, "scales")):
        _dev(t, name)
    vocab, hidden = table.shape
    out = _embed_out(ids, hidden, scales.dtype, out_dtype, table.device)
    check("qembed_w8", lib().qembed_w8(
        _ptr(ids), ids.numel(), _ptr(table), QG_LAYOUT_TILED if tiled else QG_LAYOUT_PORTABLE,
        _ptr(scales), _ptr(out), vocab, hidden, group_size, dtype_code(scales.dtype),
        dtype_code(out.dtype), _stream(table)))
    return out


# -- measurement probe -----------------------------------------------------------

def read_probe(buf: Optional[torch.Tensor], nbytes: int, out: torch.Tensor) -> torch.Tensor:
    """Stream-read the first nbytes of buf once (the HBM read ceiling); out
    (uint32/int32, >= qg_read_probe_blocks(nbytes) entries) gets one XOR word
    per workgroup.  nbytes == 0: one empty workgroup (the launch cost)."""
    _dev(out, "out")
    if buf is not None:
        _dev(buf, "buf")
        if nbytes > buf.numel() * buf.element_size():
            raise QGemmError("qg_read_probe", 2, "nbytes exceeds the buffer")
    if out.numel() < int(lib().qg_read_probe_blocks(nbytes)):
        raise QGemmError("qg_read_probe", 2, "out is too small")
    check("qg_read_probe", lib().qg_read_probe(_ptr(buf), nbytes, _ptr(out), _stream(out)))
    return out


def lds_probe(waves: int, iters: int, cycles: torch.Tensor) -> torch.Tensor:
    """LDS read loop of cycles.numel() workgroups of 64 * waves threads, one
    per CU (qg_lds_probe); cycles (int64, device) gets each workgroup's
    shader-clock cycles.  Bytes per clock per CU = iters * waves * 1024 / cycles."""
    _dev(cycles, "cycles")
    if cycles.dtype != torch.int64:
        raise QGemmError("qg_lds_probe", 4, "cycles must be int64")
    check("qg_lds_probe", lib().qg_lds_probe(waves, iters, cycles.numel(), _ptr(cycles), _stream(cycles)))
    return cycles


# -- MoE -----------------------------------------------------------------------

def moe_workspace_size(tokens: int, hidden: int, inter: int, experts: int, topk: int) -> int:
    return int(lib().qmoe_workspace_size(tokens, hidden, inter, experts, topk))


def moe_grouped(x: torch.Tensor, logits: torch.Tensor, w1_tiled: torch.Tensor, s1: torch.Tensor,
                z1: torch.Tensor, w2_tiled: torch.Tensor, s2: torch.Tensor, z2: torch.Tensor,
                topk: int, group_size: int = 64, return_routing: bool = False,
                workspace: Optional[torch.Tensor] = None, b1: Optional[torch.Tensor] = None,
                b2: Optional[torch.Tensor] = None, sel_logits: Optional[torch.Tensor] = None,
                finished: Optional[torch.Tensor] = None, renormalize: bool = True,
                out: Optional[torch.Tensor] = None):
    """Top-k MoE with SiLU-gated int4 experts.

    x [T, H]; logits fp32 [T, E]; w1_tiled [E, 2I, H/2] (tiled per expert);
    s1/z1 [E, 2I, H/g]; w2_tiled [E, H, I/2]; s2/z2 [E, H, I/g].  Optional:
    fc1 / fc2 expert biases b1 [E, 2I], b2 [E, H] (x's dtype), biased
    selection logits fp32 [T, E], a finished mask (bool/uint8 [T]) and the
    normalization mode.  Returns out [T, H] (into `out` when given) (and
    (ids int32 [T, k], weights fp32 [T, k])).
    """
    f = "qmoe_grouped"
    _need(x.dtype in _ACT and x.dim() == 2, f, _DTYPE, "x must be a 2-D bf16 or fp16 tensor [T, H]")
    T, H = x.shape
    _need(logits.dtype == torch.float32 and logits.dim() == 2, f, _DTYPE,
          "logits must be a 2-D fp32 tensor [T, E]")
    _need(logits.shape[0] == T, f, _SHAPE, f"logits must be [{T}, E] (got {list(logits.shape)})")
    E = logits.shape[1]
    _need(w1_tiled.dtype == torch.uint8 and w2_tiled.dtype == torch.uint8, f, _DTYPE,
          "w1_tiled and w2_tiled must be uint8")
    _need(w1_tiled.dim() == 3 and w1_tiled.shape[1] % 2 == 0, f, _SHAPE,
          "w1_tiled must be [E, 2I, H/2]")
    I2 = w1_tiled.shape[1]
    _need(_shape(w1_tiled) == (E, I2, H // 2), f, _SHAPE,
          f"w1_tiled must be [{E}, 2I, {H // 2}] (got {list(w1_tiled.shape)})")
    _need(_shape(w2_tiled) == (E, H, I2 // 4), f, _SHAPE,
          f"w2_tiled must be [{E}, {H}, {I2 // 4}] (got {list(w2_tiled.shape)})")
    for t, nm in ((s1, "s1"), (z1, "z1")):
        _check_groups(f, nm, t, x.dtype, I2, H, group_size, lead=(E,))
    for t, nm in ((s2, "s2"), (z2, "z2")):
        _check_groups(f, nm, t, x.dtype, H, I2 // 2, group_size, lead=(E,))
    if b1 is not None:
        _need(b1.dtype == x.dtype and _shape(b1) == (E, I2), f, _SHAPE,
              f"b1 must be [{E}, {I2}] in x's dtype")
    if b2 is not None:
        _need(b2.dtype == x.dtype and _shape(b2) == (E, H), f, _SHAPE,
              f"b2 must be [{E}, {H}] in x's dtype")
    if sel_logits is not None:
        _need(sel_logits.dtype == torch.float32 and _shape(sel_logits) == (T, E), f, _SHAPE,
              f"sel_logits must be fp32 [{T}, {E}]")
    if finished is not None:
        _need(finished.dtype in (torch.bool, torch.uint8) and _shape(finished) == (T,), f, _SHAPE,
              f"finished must be bool or uint8 [{T}]")
    _need(isinstance(topk, int) and 1 <= topk <= E, f, _SHAPE, f"topk must be in [1, {E}]")
    if out is not None:
        _need(out.dtype == x.dtype and _shape(out) == (T, H), f, _SHAPE,
              f"out must be [{T}, {H}] in x's dtype")
        _dev(out, "out")
    for t, nm in ((x, "x"), (logits, "logits"), (w1_tiled, "w1_tiled"), (s1, "s1"), (z1, "z1"),
                  (w2_tiled, "w2_tiled"), (s2, "s2"), (z2, "z2")):
        _dev(t, nm)
    for t, nm in ((b1, "b1"), (b2, "b2"), (sel_logits, "sel_logits"), (finished, "finished")):
        if t is not None:
            _dev(t, nm)
    if finished is not None and finished.dtype == torch.bool:
        finished = finished.view(torch.uint8)
    inter = I2 // 2
    if out is None:
        out = torch.empty_like(x)
    ids = torch.empty((T, topk), dtype=torch.int32, device=x.device) if return_routing else None
    wts = torch.empty((T, topk), dtype=torch.float32, device=x.device) if return_routing else None
    need = moe_workspace_size(T, H, inter, E, topk)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    _dev(workspace, "workspace")
    if b1 is None and b2 is None and sel_logits is None and finished is None and renormalize:
        check("qmoe_grouped", lib().qmoe_grouped(
            _ptr(x), _ptr(logits), _ptr(w1_tiled), _ptr(s1), _ptr(z1), _ptr(w2_tiled), _ptr(s2),
            _ptr(z2), _ptr(out), T, H, inter, E, topk, group_size, dtype_code(x.dtype), _ptr(ids),
            _ptr(wts), _ptr(workspace), workspace.numel(), _stream(x)))
    else:
        check("qmoe_grouped_ex", lib().qmoe_grouped_ex(
            _ptr(x), _ptr(logits), _ptr(sel_logits), _ptr(finished), _ptr(w1_tiled), _ptr(s1),
            _ptr(z1), _ptr(b1), _ptr(w2_tiled), _ptr(s2), _ptr(z2), _ptr(b2), _ptr(out), T, H,
            inter, E, topk, group_size, QG_MOE_RENORMALIZE if renormalize else QG_MOE_NORM_NONE,
            dtype_code(x.dtype), _ptr(ids), _ptr(wts), _ptr(workspace), workspace.numel(),
            _stream(x)))
    if return_routing:
        return out, ids, wts
    return out


def moe_grouped_noalloc(x: torch.Tensor, logits: torch.Tensor, w1_tiled: torch.Tensor,
                        s1: torch.Tensor, z1: torch.Tensor, w2_tiled: torch.Tensor,
                        s2: torch.Tensor, z2: torch.Tensor, topk: int, group_size: int,
                        out: torch.Tensor, ids: Optional[torch.Tensor] = None,
                        wts: Optional[torch.Tensor] = None) -> torch.Tensor:
    """moe_grouped into caller-given `out` (and optional `ids` int32 [T, k],
    `wts` fp32 [T, k]) on the library's device scratch: no workspace, no
    allocation (qmoe_grouped_noalloc; at most 64 MiB of workspace needed)."""
    f = "qmoe_grouped_noalloc"
    _need(x.dtype in _ACT and x.dim() == 2, f, _DTYPE, "x must be a 2-D bf16 or fp16 tensor [T, H]")
    T, H = x.shape
    _need(logits.dtype == torch.float32 and logits.dim() == 2 and logits.shape[0] == T, f, _SHAPE,
          f"logits must be fp32 [{T}, E]")
    E = logits.shape[1]
    _need(w1_tiled.dtype == torch.uint8 and w1_tiled.dim() == 3, f, _DTYPE, "w1_tiled must be uint8 [E, 2I, H/2]")
    I2 = w1_tiled.shape[1]
    _need(_shape(w1_tiled) == (E, I2, H // 2) and I2 % 2 == 0, f, _SHAPE, "w1_tiled must be [E, 2I, H/2]")
    _need(w2_tiled.dtype == torch.uint8 and _shape(w2_tiled) == (E, H, I2 // 4), f, _SHAPE,
          "w2_tiled must be uint8 [E, H, I/2]")
    for t, nm in ((s1, "s1"), (z1, "z1")):
        _check_groups(f, nm, t, x.dtype, I2, H, group_size, lead=(E,))
    for t, nm in ((s2, "s2"), (z2, "z2")):
        _check_groups(f, nm, t, x.dtype, H, I2 // 2, group_size, lead=(E,))
    _need(out.dtype == x.dtype and _shape(out) == (T, H), f, _SHAPE, f"out must be [{T}, {H}]")
    if ids is not None:
        _need(ids.dtype == torch.int32 and _shape(ids) == (T, topk), f, _SHAPE, f"ids must be int32 [{T}, {topk}]")
    if wts is not None:
        _need(wts.dtype == torch.float32 and _shape(wts) == (T, topk), f, _SHAPE,
              f"wts must be fp32 [{T}, {topk}]")
    for t, nm in ((x, "x"), (logits, "logits"), (w1_tiled, "w1_tiled"), (s1, "s1"), (z1, "z1"),
                  (w2_tiled, "w2_tiled"), (s2, "s2"), (z2, "z2"), (out, "out"), (ids, "ids"),
                  (wts, "wts")):
        if t is not None:
            _dev(t, nm)
    check(f, lib().qmoe_grouped_noalloc(
        _ptr(x), _ptr(logits), _ptr(w1_tiled), _ptr(s1), _ptr(z1), _ptr(w2_tiled), _ptr(s2),
        _ptr(z2), _ptr(out), T, H, I2 // 2, E, topk, group_size, dtype_code(x.dtype), _ptr(ids),
        _ptr(wts), _stream(x)))
    return out
