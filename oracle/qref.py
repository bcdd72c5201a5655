"""Python face of the CPU oracle (``qref.c``), plus its build step.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares no code
with the HIP library and never imports it.

All arithmetic lives in ``qref.c`` (plain C, double accumulation); this file
only marshals numpy arrays.  16-bit floats cross as raw ``uint16`` bit
patterns; dtype codes are 0 = none, 1 = bf16, 2 = fp16.

What each function computes, and which page passage defines it, is stated in
``qref.c``.  Parity pins (tests that tie the oracle to the pages and to
mathematics rather than to itself) live in ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

__all__ = [
    "NONE", "BF16", "FP16", "build", "lib", "bf16_to_f32", "f16_to_f32", "f32_to_bf16",
    "f32_to_f16", "pack4", "unpack4", "quantize4", "dequant4", "dequant8", "gemm_w4", "gemm_w8",
    "gemm_w4_at", "gemm_w8_at", "gemm_w8a8", "moe_route", "moe", "threads", "embed4", "embed8",
    "gemm_w4_f32acc", "gemm_w8_f32acc", "set_threads", "team_size",
]

NONE, BF16, FP16 = 0, 1, 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qref.c")
_LIB = os.path.join(_HERE, "libqref.so")
_lock = threading.Lock()
_lib = None

# -ffp-contract=off: no fused multiply-add contraction, so every operation
# rounds exactly as written.  No -ffast-math: no reassociation.
_CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wno-unknown-pragmas"]


def build(force: bool = True) -> str:
    """Compile ``qref.c`` into ``libqref.so`` next to it (gcc, OpenMP)."""
    global _lib
    with _lock:
        if force or not os.path.exists(_LIB):
            tmp = _LIB + ".tmp%d" % os.getpid()
            subprocess.check_call(["gcc", *_CFLAGS, _SRC, "-o", tmp, "-lm"])
            os.replace(tmp, _LIB)
            _lib = None
    return _LIB


_P = ctypes.c_void_p
_I = ctypes.c_int64
_INT = ctypes.c_int

_SIGS = {
    "qref_bf16_to_f32": (ctypes.c_float, [ctypes.c_uint16]),
    "qref_f16_to_f32": (ctypes.c_float, [ctypes.c_uint16]),
    "qref_f32_to_bf16": (ctypes.c_uint16, [ctypes.c_float]),
    "qref_f32_to_f16": (ctypes.c_uint16, [ctypes.c_float]),
    "qref_pack4": (None, [_P, _P, _I, _I]),
    "qref_unpack4": (None, [_P, _P, _I, _I]),
    "qref_quantize4": (None, [_P, _I, _I, _I, _P, _P, _P]),
    "qref_dequant4": (None, [_P, _P, _P, _I, _I, _I, _INT, _P]),
    "qref_dequant8": (None, [_P, _P, _I, _I, _I, _INT, _P]),
    "qref_gemm_w4": (None, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _INT, _INT, _P]),
    "qref_gemm_w8": (None, [_P, _P, _P, _P, _I, _I, _I, _I, _INT, _INT, _P]),
    "qref_gemm_w4_f32acc": (None, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _INT, _INT, _P]),
    "qref_gemm_w8_f32acc": (None, [_P, _P, _P, _P, _I, _I, _I, _I, _INT, _INT, _P]),
    "qref_threads": (_INT, []),
    "qref_set_threads": (None, [_INT]),
    "qref_team_size": (_INT, []),
    "qref_gemm_w4_at": (None, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _INT, _INT, _P, _P, _I, _P]),
    "qref_gemm_w8_at": (None, [_P, _P, _P, _P, _I, _I, _I, _I, _INT, _INT, _P, _P, _I, _P]),
    "qref_embed4": (None, [_P, _I, _P, _P, _P, _I, _I, _I, _INT, _P]),
    "qref_embed8": (None, [_P, _I, _P, _P, _I, _I, _I, _INT, _P]),
    "qref_gemm_w8a8": (None, [_P, _P, _P, _INT, _P, _INT, _I, _I, _I, _P, _P]),
    "qref_moe_route": (None, [_P, _I, _I, _I, _P, _P]),
    "qref_moe_route_ex": (None, [_P, _P, _P, _I, _I, _I, _INT, _P, _P]),
    "qref_moe_ex": (None, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I,
                           _INT, _INT, _P, _I, _P, _P, _P]),
    "qref_moe": (None, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _INT,
                        _P, _I, _P, _P, _P]),
}


def lib():
    """The loaded oracle library (built on first use if absent)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        with _lock:
            if _lib is None:
                handle = ctypes.CDLL(_LIB)
                for name, (res, args) in _SIGS.items():
                    fn = getattr(handle, name)
                    fn.restype = res
                    fn.argtypes = args
                _lib = handle
    return _lib


def threads() -> int:
    """OpenMP threads the oracle's parallel loops will ask for
    (omp_get_max_threads() inside the library)."""
    return int(lib().qref_threads())


def set_threads(n: int) -> None:
    """Ask for n threads in the oracle's parallel loops from now on."""
    lib().qref_set_threads(int(n))


def team_size() -> int:
    """Threads a parallel region of the oracle actually runs on."""
    return int(lib().qref_team_size())


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=dtype)


# -- scalar / elementwise conversions (vectorised over numpy arrays) -------

def bf16_to_f32(bits):
    f = lib().qref_bf16_to_f32
    b = np.asarray(bits, dtype=np.uint16)
    return np.array([f(int(v)) for v in b.ravel()], dtype=np.float32).reshape(b.shape)


def f16_to_f32(bits):
    f = lib().qref_f16_to_f32
    b = np.asarray(bits, dtype=np.uint16)
    return np.array([f(int(v)) for v in b.ravel()], dtype=np.float32).reshape(b.shape)


def f32_to_bf16(x):
    f = lib().qref_f32_to_bf16
    a = np.asarray(x, dtype=np.float32)
    return np.array([f(float(v)) for v in a.ravel()], dtype=np.uint16).reshape(a.shape)


def f32_to_f16(x):
    f = lib().qref_f32_to_f16
    a = np.asarray(x, dtype=np.float32)
    return np.array([f(float(v)) for v in a.ravel()], dtype=np.uint16).reshape(a.shape)


# -- packing ----------------------------------------------------------------

def pack4(codes):
    """[N, K] codes in [0, 15] -> [N, K/2] uint8, low nibble = even k."""
    q = _c(codes, np.int32)
    n, k = q.shape
    out = np.empty((n, k // 2), dtype=np.uint8)
    lib().qref_pack4(_ptr(q), _ptr(out), n, k)
    return out


def unpack4(packed):
    """[N, K/2] uint8 -> [N, K] int32 codes."""
    p = _c(packed, np.uint8)
    n, half = p.shape
    out = np.empty((n, half * 2), dtype=np.int32)
    lib().qref_unpack4(_ptr(p), _ptr(out), n, half * 2)
    return out


# -- quantization ---------------------------------------------------------------

def quantize4(w, group):
    """Groupwise min/max 4-bit quantization of fp32 [N, K].

    Returns (packed uint8 [N, K/2], scale fp32 [N, K/g], zero fp32 [N, K/g]).
    """
    x = _c(w, np.float32)
    n, k = x.shape
    assert k % group == 0 and k % 2 == 0
    packed = np.zeros((n, k // 2), dtype=np.uint8)
    scale = np.empty((n, k // group), dtype=np.float32)
    zero = np.empty((n, k // group), dtype=np.float32)
    lib().qref_quantize4(_ptr(x), n, k, group, _ptr(packed), _ptr(scale), _ptr(zero))
    return packed, scale, zero


# -- dequantization -----------------------------------------------------------

def dequant4(packed, scale, zero, group, dtype=BF16):
    """fp32 [N, K] with w = (q - 8) * scale + zero per K-group."""
    p = _c(packed, np.uint8)
    n, half = p.shape
    k = half * 2
    s = _c(scale, np.uint16)
    z = _c(zero, np.uint16)
    out = np.empty((n, k), dtype=np.float32)
    lib().qref_dequant4(_ptr(p), _ptr(s), _ptr(z), n, k, group, dtype, _ptr(out))
    return out


def dequant8(codes, scale, group=-1, dtype=FP16):
    """fp32 [N, K] with w = q * scale (per channel for group -1)."""
    q = _c(codes, np.int8)
    n, k = q.shape
    s = _c(scale, np.uint16)
    out = np.empty((n, k), dtype=np.float32)
    lib().qref_dequant8(_ptr(q), _ptr(s), n, k, group, dtype, _ptr(out))
    return out


def embed4(ids, packed, scale, zero, group, dtype=BF16):
    """fp32 [T, hidden]: row ids[t] of the int4 table (portable [vocab,
    hidden/2] codes), dequantized; rows of zeros for ids outside the table."""
    i = _c(np.asarray(ids).reshape(-1), np.int32)
    p = _c(packed, np.uint8)
    vocab, half = p.shape
    hidden = half * 2
    out = np.empty((i.size, hidden), dtype=np.float32)
    lib().qref_embed4(_ptr(i), i.size, _ptr(p), _ptr(_c(scale, np.uint16)), _ptr(_c(zero, np.uint16)),
                      vocab, hidden, group, dtype, _ptr(out))
    return out


def embed8(ids, codes, scale, group=-1, dtype=FP16):
    """fp32 [T, hidden]: row ids[t] of the int8 table [vocab, hidden],
    dequantized; rows of zeros for ids outside the table."""
    i = _c(np.asarray(ids).reshape(-1), np.int32)
    q = _c(codes, np.int8)
    vocab, hidden = q.shape
    out = np.empty((i.size, hidden), dtype=np.float32)
    lib().qref_embed8(_ptr(i), i.size, _ptr(q), _ptr(_c(scale, np.uint16)), vocab, hidden, group,
                      dtype, _ptr(out))
    return out


# -- GEMM ---------------------------------------------------------------------

def gemm_w4(A, packed, scale, zero, group, dtype=BF16, bias=None, bias_dtype=NONE):
    """C = A @ dequant4(B)^T (+ bias) in double, [M, N]."""
    a = _c(A, np.uint16)
    p = _c(packed, np.uint8)
    m, k = a.shape
    n = p.shape[0]
    assert p.shape[1] * 2 == k
    out = np.empty((m, n), dtype=np.float64)
    bb = _c(bias, np.uint16)
    lib().qref_gemm_w4(_ptr(a), _ptr(p), _ptr(_c(scale, np.uint16)), _ptr(_c(zero, np.uint16)),
                       _ptr(bb), m, n, k, group, dtype, bias_dtype if bb is not None else NONE,
                       _ptr(out))
    return out


def gemm_w8(A, codes, scale, group=-1, dtype=FP16, bias=None, bias_dtype=NONE):
    """C = A @ dequant8(B)^T (+ bias) in double, [M, N]."""
    a = _c(A, np.uint16)
    q = _c(codes, np.int8)
    m, k = a.shape
    n = q.shape[0]
    assert q.shape[1] == k
    out = np.empty((m, n), dtype=np.float64)
    bb = _c(bias, np.uint16)
    lib().qref_gemm_w8(_ptr(a), _ptr(q), _ptr(_c(scale, np.uint16)), _ptr(bb), m, n, k, group,
                       dtype, bias_dtype if bb is not None else NONE, _ptr(out))
    return out


def gemm_w4_f32acc(A, packed, scale, zero, group, dtype=BF16, bias=None, bias_dtype=NONE):
    """The w4 GEMM with fp32 accumulation (the timed CPU baseline), float32 [M, N]."""
    a = _c(A, np.uint16)
    p = _c(packed, np.uint8)
    m, k = a.shape
    n = p.shape[0]
    assert p.shape[1] * 2 == k
    out = np.empty((m, n), dtype=np.float32)
    bb = _c(bias, np.uint16)
    lib().qref_gemm_w4_f32acc(_ptr(a), _ptr(p), _ptr(_c(scale, np.uint16)),
                              _ptr(_c(zero, np.uint16)), _ptr(bb), m, n, k, group, dtype,
                              bias_dtype if bb is not None else NONE, _ptr(out))
    return out


def gemm_w8_f32acc(A, codes, scale, group=-1, dtype=FP16, bias=None, bias_dtype=NONE):
    """The w8 GEMM with fp32 accumulation, float32 [M, N]."""
    a = _c(A, np.uint16)
    q = _c(codes, np.int8)
    m, k = a.shape
    n = q.shape[0]
    assert q.shape[1] == k
    out = np.empty((m, n), dtype=np.float32)
    bb = _c(bias, np.uint16)
    lib().qref_gemm_w8_f32acc(_ptr(a), _ptr(q), _ptr(_c(scale, np.uint16)), _ptr(bb), m, n, k,
                              group, dtype, bias_dtype if bb is not None else NONE, _ptr(out))
    return out


def gemm_w4_at(A, packed, scale, zero, group, rows, cols, dtype=BF16, bias=None, bias_dtype=NONE):
    """The w4 GEMM evaluated only at the (rows[i], cols[i]) pairs."""
    a = _c(A, np.uint16)
    p = _c(packed, np.uint8)
    m, k = a.shape
    n = p.shape[0]
    r = _c(rows, np.int64)
    c = _c(cols, np.int64)
    assert r.shape == c.shape
    assert (r >= 0).all() and (r < m).all() and (c >= 0).all() and (c < n).all()
    out = np.empty(r.shape, dtype=np.float64)
    bb = _c(bias, np.uint16)
    lib().qref_gemm_w4_at(_ptr(a), _ptr(p), _ptr(_c(scale, np.uint16)), _ptr(_c(zero, np.uint16)),
                          _ptr(bb), m, n, k, group, dtype,
                          bias_dtype if bb is not None else NONE, _ptr(r), _ptr(c), r.size,
                          _ptr(out))
    return out


def gemm_w8_at(A, codes, scale, rows, cols, group=-1, dtype=FP16, bias=None, bias_dtype=NONE):
    """The w8 GEMM evaluated only at the (rows[i], cols[i]) pairs."""
    a = _c(A, np.uint16)
    q = _c(codes, np.int8)
    m, k = a.shape
    n = q.shape[0]
    r = _c(rows, np.int64)
    c = _c(cols, np.int64)
    assert (r >= 0).all() and (r < m).all() and (c >= 0).all() and (c < n).all()
    out = np.empty(r.shape, dtype=np.float64)
    bb = _c(bias, np.uint16)
    lib().qref_gemm_w8_at(_ptr(a), _ptr(q), _ptr(_c(scale, np.uint16)), _ptr(bb), m, n, k, group,
                          dtype, bias_dtype if bb is not None else NONE, _ptr(r), _ptr(c), r.size,
                          _ptr(out))
    return out


# -- W8A8 ---------------------------------------------------------------------

def gemm_w8a8(A, B, alpha_row, alpha_col):
    """int8 A [M, K] x int8 B [N, K]: (exact int64 sums [M, N], double C [M, N]).

    alpha_row has M entries (per token) or 1 (per tensor); alpha_col N or 1.
    """
    a = _c(A, np.int8)
    b = _c(B, np.int8)
    m, k = a.shape
    n = b.shape[0]
    assert b.shape[1] == k
    ar = _c(np.atleast_1d(alpha_row), np.float32)
    ac = _c(np.atleast_1d(alpha_col), np.float32)
    per_token, per_channel = int(ar.size == m and m > 1), int(ac.size == n and n > 1)
    assert ar.size in (1, m) and ac.size in (1, n)
    acc = np.empty((m, n), dtype=np.int64)
    out = np.empty((m, n), dtype=np.float64)
    lib().qref_gemm_w8a8(_ptr(a), _ptr(b), _ptr(ar), per_token, _ptr(ac), per_channel, m, n, k,
                         _ptr(acc), _ptr(out))
    return acc, out


# -- MoE ----------------------------------------------------------------------

def moe_route(logits, topk, sel_logits=None, finished=None, renormalize=True):
    """Top-k expert ids (int32 [T, k], descending selection logit, ties to the
    lower id) and their weights (double [T, k]): softmax of the gating logits
    over the selected experts (renormalize) or over all of them.  sel_logits:
    the biased logits that choose the experts (default: the gating logits);
    finished rows: ids -1, weights 0."""
    lg = _c(logits, np.float32)
    t, e = lg.shape
    ids = np.empty((t, topk), dtype=np.int32)
    w = np.empty((t, topk), dtype=np.float64)
    lib().qref_moe_route_ex(_ptr(lg), _ptr(_c(sel_logits, np.float32)), _ptr(_c(finished, np.uint8)),
                            t, e, topk, int(bool(renormalize)), _ptr(ids), _ptr(w))
    return ids, w


def moe(x, logits, w1, s1, z1, w2, s2, z2, topk, group, dtype=BF16, tokens=None, b1=None, b2=None,
        sel_logits=None, finished=None, renormalize=True):
    """Top-k MoE with SiLU-gated experts, in double.

    x [T, H] (16-bit bits), logits fp32 [T, E], w1 [E, 2I, H/2] u8,
    s1/z1 [E, 2I, H/g], w2 [E, H, I/2] u8, s2/z2 [E, H, I/g]; optional fc1 /
    fc2 biases b1 [E, 2I], b2 [E, H] (16-bit bits), selection logits,
    finished rows (zero output) and the normalization mode (see moe_route).
    ``tokens`` selects which rows of the output to compute (default: all).
    Returns (out [len(tokens), H] double, ids [T, k] int32, weights [T, k]).
    """
    xx = _c(x, np.uint16)
    lg = _c(logits, np.float32)
    W1 = _c(w1, np.uint8)
    W2 = _c(w2, np.uint8)
    t, h = xx.shape
    e = lg.shape[1]
    two_i = W1.shape[1]
    inter = two_i // 2
    assert W1.shape == (e, two_i, h // 2) and W2.shape == (e, h, inter // 2)
    sel = np.arange(t, dtype=np.int64) if tokens is None else _c(tokens, np.int64)
    out = np.empty((sel.size, h), dtype=np.float64)
    ids = np.empty((t, topk), dtype=np.int32)
    wts = np.empty((t, topk), dtype=np.float64)
    lib().qref_moe_ex(_ptr(xx), _ptr(lg), _ptr(_c(sel_logits, np.float32)),
                      _ptr(_c(finished, np.uint8)), _ptr(W1), _ptr(_c(s1, np.uint16)),
                      _ptr(_c(z1, np.uint16)), _ptr(_c(b1, np.uint16)), _ptr(W2),
                      _ptr(_c(s2, np.uint16)), _ptr(_c(z2, np.uint16)), _ptr(_c(b2, np.uint16)),
                      t, h, inter, e, topk, group, int(bool(renormalize)), dtype, _ptr(sel), sel.size,
                      _ptr(ids), _ptr(wts), _ptr(out))
    return out, ids, wts
