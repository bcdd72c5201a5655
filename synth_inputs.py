"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the
benchmark.

This module draws random numbers and nothing else: it holds none of the
method's arithmetic (no packing, dequantization or products).  Random 4-bit
codes are drawn directly as uniform random bytes -- two independent uniform
nibbles per byte -- which is exactly the portable packed layout of uniform
codes in [0, 15].  Floats are drawn in fp32 and rounded to bf16/fp16 by torch's
round-to-nearest-even cast, then handed out as raw uint16 bit patterns.

Draw order inside one problem is fixed: codes, scales, zeros, bias, A, logits.
Weights and activations use separate seeds, so an M sweep shares its weights.

Workload distributions (per the problem statements being reproduced):
  W4A16:  codes U{0..15}; scale U[0.005, 0.02]; zero N(0, 0.01); A N(0, 1);
          bias (when present) N(0, 0.02) in fp16; bf16 everything else.
  W8A16:  codes U{-127..127}; per-channel scale U[0.001, 0.01]; no zero;
          A N(0, 1); fp16 everything.
  MoE:    x N(0, 1) bf16; gating logits N(0, 1) fp32; expert weights as W4A16.
"""
from __future__ import annotations

import zlib
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

NONE, BF16, FP16 = 0, 1, 2
_TORCH = {BF16: torch.bfloat16, FP16: torch.float16}


def seed_of(*parts) -> int:
    """Stable 31-bit seed from a tuple of names and sizes."""
    return zlib.crc32(repr(parts).encode()) & 0x7FFFFFFF


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator()
    g.manual_seed(int(seed))
    return g


def _bits(t: torch.Tensor, dtype: int) -> np.ndarray:
    return t.to(_TORCH[dtype]).contiguous().view(torch.int16).numpy().view(np.uint16)


def _uniform(g, shape, lo, hi):
    return torch.rand(shape, generator=g, dtype=torch.float32) * (hi - lo) + lo


def _normal(g, shape, std):
    return torch.randn(shape, generator=g, dtype=torch.float32) * std


@dataclass
class W4Problem:
    m: int
    n: int
    k: int
    group: int
    dtype: int
    A: np.ndarray              # uint16 bits [m, k]
    packed: np.ndarray         # uint8 [n, k/2]
    scale: np.ndarray          # uint16 bits [n, k/group]
    zero: np.ndarray           # uint16 bits [n, k/group]
    bias: Optional[np.ndarray] = None   # uint16 bits [n]
    bias_dtype: int = NONE


@dataclass
class W8Problem:
    m: int
    n: int
    k: int
    group: int
    dtype: int
    A: np.ndarray              # uint16 bits [m, k]
    codes: np.ndarray          # int8 [n, k]
    scale: np.ndarray          # uint16 bits [n] (group -1) or [n, k/group]
    bias: Optional[np.ndarray] = None
    bias_dtype: int = NONE


def w4_weights(n, k, group, seed, dtype=BF16, scale_range=(0.005, 0.02), zero_std=0.01,
               bias_dtype=NONE, bias_std=0.02):
    g = _gen(seed)
    packed = torch.randint(0, 256, (n, k // 2), generator=g, dtype=torch.uint8).numpy()
    sshape = (n,) if group in (-1, k) else (n, k // group)   # -1: one per channel
    scale = _bits(_uniform(g, sshape, *scale_range), dtype)
    zero = _bits(_normal(g, sshape, zero_std), dtype)
    bias = _bits(_normal(g, (n,), bias_std), bias_dtype) if bias_dtype != NONE else None
    return packed, scale, zero, bias


def activations(m, k, seed, dtype=BF16, std=1.0):
    g = _gen(seed)
    return _bits(_normal(g, (m, k), std), dtype)


def w4_problem(m, n, k, group, tag="w4", dtype=BF16, bias_dtype=NONE, **kw) -> W4Problem:
    packed, scale, zero, bias = w4_weights(n, k, group, seed_of(tag, "w", n, k, group), dtype,
                                           bias_dtype=bias_dtype, **kw)
    A = activations(m, k, seed_of(tag, "a", m, k), dtype)
    return W4Problem(m, n, k, group, dtype, A, packed, scale, zero, bias, bias_dtype)


def w8_weights(n, k, group, seed, dtype=FP16, scale_range=(0.001, 0.01), bias_dtype=NONE,
               bias_std=0.02):
    g = _gen(seed)
    codes = torch.randint(-127, 128, (n, k), generator=g, dtype=torch.int8).numpy()
    sshape = (n,) if group in (-1, k) else (n, k // group)
    scale = _bits(_uniform(g, sshape, *scale_range), dtype)
    bias = _bits(_normal(g, (n,), bias_std), bias_dtype) if bias_dtype != NONE else None
    return codes, scale, bias


def w8_problem(m, n, k, group=-1, tag="w8", dtype=FP16, bias_dtype=NONE, **kw) -> W8Problem:
    codes, scale, bias = w8_weights(n, k, group, seed_of(tag, "w", n, k, group), dtype,
                                    bias_dtype=bias_dtype, **kw)
    A = activations(m, k, seed_of(tag, "a", m, k), dtype)
    return W8Problem(m, n, k, group, dtype, A, codes, scale, bias, bias_dtype)


# -- W8A8: int8 activation and weight codes, fp32 row / column scales ----------

@dataclass
class W8A8Problem:
    m: int
    n: int
    k: int
    A: np.ndarray           # int8 [m, k]
    B: np.ndarray           # int8 [n, k]
    alpha_row: np.ndarray   # fp32 [m] (per token) or [1]
    alpha_col: np.ndarray   # fp32 [n] (per channel) or [1]


def _codes8(g, shape, lo, hi):
    return torch.randint(lo, hi + 1, shape, generator=g, dtype=torch.int32).to(torch.int8).numpy()


def w8a8_problem(m, n, k, per_token, per_channel, tag="w8a8", code_range=(-127, 127),
                 row_range=(0.005, 0.05), col_range=(0.001, 0.01), scales=None) -> W8A8Problem:
    """Symmetric int8 codes uniform in code_range for both operands; scales
    uniform in the given ranges, or drawn from the list `scales` (e.g. powers
    of two) when given."""
    gw = _gen(seed_of(tag, "w", n, k, per_channel, code_range))
    B = _codes8(gw, (n, k), *code_range)
    nc = n if per_channel else 1
    ga = _gen(seed_of(tag, "a", m, k, per_token, code_range))
    A = _codes8(ga, (m, k), *code_range)
    nr = m if per_token else 1
    if scales is None:
        col = _uniform(gw, (nc,), *col_range).numpy()
        row = _uniform(ga, (nr,), *row_range).numpy()
    else:
        sv = torch.tensor(scales, dtype=torch.float32)
        col = sv[torch.randint(0, len(scales), (nc,), generator=gw)].numpy()
        row = sv[torch.randint(0, len(scales), (nr,), generator=ga)].numpy()
    return W8A8Problem(m, n, k, A, B, row.astype(np.float32), col.astype(np.float32))


# -- inputs whose exact product is representable -------------------------------
# Activations in {-2..2}, scales in {1, 1/2, 1/4}, zeros multiples of 1/4 in
# [-1, 1], bias multiples of 1/4: every partial sum is a multiple of 2^-2 well
# below 2^24 in magnitude, so any fp32 summation order gives the exact value.

def w4_exact_problem(m, n, k, group, seed, dtype=BF16, bias_dtype=NONE,
                     zeros=True) -> W4Problem:
    """group -1: one scale (and zero) per channel; zeros=False: no zeros
    (scale-only weights), `zero` is None."""
    g = _gen(seed)
    packed = torch.randint(0, 256, (n, k // 2), generator=g, dtype=torch.uint8).numpy()
    sshape = (n,) if group in (-1, k) else (n, k // group)
    sexp = torch.randint(0, 3, sshape, generator=g)
    scale = _bits(torch.pow(2.0, -sexp.float()), dtype)
    zero = _bits(torch.randint(-4, 5, sshape, generator=g).float() / 4.0, dtype)
    if not zeros:
        zero = None
    bias = None
    if bias_dtype != NONE:
        bias = _bits(torch.randint(-8, 9, (n,), generator=g).float() / 4.0, bias_dtype)
    A = _bits(torch.randint(-2, 3, (m, k), generator=g).float(), dtype)
    return W4Problem(m, n, k, group, dtype, A, packed, scale, zero, bias, bias_dtype)


def w8_exact_problem(m, n, k, seed, dtype=FP16, bias_dtype=NONE, group=-1) -> W8Problem:
    """A in {-1, 0, 1}, scales 2^-4 .. 2^-6 (per channel, or per K-group for
    group 64 / 128): |C| < 2^15, every partial sum a multiple of 2^-6, exact."""
    g = _gen(seed)
    codes = torch.randint(-128, 128, (n, k), generator=g, dtype=torch.int8).numpy()
    sshape = (n,) if group in (-1, k) else (n, k // group)
    sexp = torch.randint(4, 7, sshape, generator=g)
    scale = _bits(torch.pow(2.0, -sexp.float()), dtype)
    bias = None
    if bias_dtype != NONE:
        bias = _bits(torch.randint(-8, 9, (n,), generator=g).float() / 4.0, bias_dtype)
    A = _bits(torch.randint(-1, 2, (m, k), generator=g).float(), dtype)
    return W8Problem(m, n, k, group, dtype, A, codes, scale, bias, bias_dtype)


# -- MoE ---------------------------------------------------------------------------

@dataclass
class MoEProblem:
    tokens: int
    hidden: int
    inter: int
    experts: int
    topk: int
    group: int
    dtype: int
    x: np.ndarray          # uint16 [T, H]
    logits: np.ndarray     # float32 [T, E]
    w1: np.ndarray         # uint8 [E, 2I, H/2]
    s1: np.ndarray         # uint16 [E, 2I, H/g]
    z1: np.ndarray
    w2: np.ndarray         # uint8 [E, H, I/2]
    s2: np.ndarray         # uint16 [E, H, I/g]
    z2: np.ndarray
    extra: dict = field(default_factory=dict)


def moe_problem(tokens, hidden, inter, experts, topk, group=64, tag="moe", dtype=BF16,
                scale_range=(0.005, 0.02), zero_std=0.01, logit_std=1.0) -> MoEProblem:
    g = _gen(seed_of(tag, "w", hidden, inter, experts, group))
    w1 = torch.randint(0, 256, (experts, 2 * inter, hidden // 2), generator=g,
                       dtype=torch.uint8).numpy()
    s1 = _bits(_uniform(g, (experts, 2 * inter, hidden // group), *scale_range), dtype)
    z1 = _bits(_normal(g, (experts, 2 * inter, hidden // group), zero_std), dtype)
    w2 = torch.randint(0, 256, (experts, hidden, inter // 2), generator=g,
                       dtype=torch.uint8).numpy()
    s2 = _bits(_uniform(g, (experts, hidden, inter // group), *scale_range), dtype)
    z2 = _bits(_normal(g, (experts, hidden, inter // group), zero_std), dtype)
    ga = _gen(seed_of(tag, "a", tokens, hidden, experts))
    x = _bits(_normal(ga, (tokens, hidden), 1.0), dtype)
    logits = _normal(ga, (tokens, experts), logit_std).numpy()
    return MoEProblem(tokens, hidden, inter, experts, topk, group, dtype, x, logits,
                      w1, s1, z1, w2, s2, z2)


def moe_extras(p: MoEProblem, tag="moe-extras", bias_std=0.02, gate_bias_std=0.5,
               finished_frac=0.1):
    """Inputs of the MoE's optional parts: fc1 / fc2 expert biases (activation
    dtype, N(0, bias_std)), selection logits = gating logits + a per-expert
    bias drawn N(0, gate_bias_std) (the 'gating output with bias' input), and
    a finished-row mask with about finished_frac of the rows set."""
    g = _gen(seed_of(tag, p.tokens, p.hidden, p.inter, p.experts))
    b1 = _bits(_normal(g, (p.experts, 2 * p.inter), bias_std), p.dtype)
    b2 = _bits(_normal(g, (p.experts, p.hidden), bias_std), p.dtype)
    gbias = _normal(g, (1, p.experts), gate_bias_std)
    sel = (torch.from_numpy(p.logits) + gbias).numpy().astype(np.float32)
    finished = (torch.rand((p.tokens,), generator=g) < finished_frac).to(torch.uint8).numpy()
    return b1, b2, sel, finished
