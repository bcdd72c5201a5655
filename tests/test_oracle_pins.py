"""Pins that tie the CPU oracle to the pages and to mathematics.

None of these compares the oracle with itself: each checks it against a
worked example (tests/golden), a library routine it must agree with, a closed
form, or an invariant the definition implies.  A dropped term, a wrong sign, a
swapped nibble or a transposed operand fails at least one of them.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si

BF16, FP16 = oracle.BF16, oracle.FP16


def bf16_bits(x):
    return torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def f16_bits(x):
    return np.asarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


# -- 16-bit float conversions vs library routines ------------------------------

def test_bf16_widen_all_patterns_match_torch():
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.bf16_to_f32(allbits)
    ref = torch.from_numpy(allbits.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    same = (ours.view(np.uint32) == ref.view(np.uint32)) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()


def test_f16_widen_all_patterns_match_numpy():
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.f16_to_f32(allbits)
    ref = allbits.view(np.float16).astype(np.float32)
    same = (ours.view(np.uint32) == ref.view(np.uint32)) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()


def _rounding_cases(rng):
    x = rng.standard_normal(20000).astype(np.float32) * np.float32(3.0)
    # exact ties for bf16: low 16 bits == 0x8000 with both parities of the kept lsb
    ties = (rng.integers(0x3F000000, 0x47000000, 4000, dtype=np.uint32) & ~np.uint32(0xFFFF)) | np.uint32(0x8000)
    # fp16 ties: values k + 0.5 ulp in several binades, incl. subnormal range
    f16 = np.arange(1, 65504, 97, dtype=np.float32)
    halfway = np.concatenate([f16 + 0.5, (f16 + 0.5) * np.float32(2.0 ** -14), (f16 + 0.5) * np.float32(2.0 ** -24)])
    big = np.array([65504, 65519, 65520, 65536, 1e9, -65520, 6e-8, 2.9e-8, 3.0e-8, 0.0, -0.0], dtype=np.float32)
    return np.concatenate([x, ties.view(np.float32), halfway.astype(np.float32), big, -x[:1000]])


def test_f32_to_bf16_matches_torch_rne():
    x = _rounding_cases(np.random.default_rng(1))
    ours = oracle.f32_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (ours == ref).all()


def test_f32_to_f16_matches_numpy_rne():
    x = _rounding_cases(np.random.default_rng(2))
    ours = oracle.f32_to_f16(x)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert (ours == ref).all()


# -- nibble packing (worked bytes from the stated byte formula) ---------------

def test_pack_worked_bytes():
    assert oracle.pack4([[1, 2]]).tolist() == [[0x21]]          # low nibble = even k
    assert oracle.unpack4(np.array([[0xA5]], np.uint8)).tolist() == [[5, 10]]


def test_pack_unpack_all_bytes_round_trip():
    b = np.arange(256, dtype=np.uint8).reshape(2, 128)
    assert (oracle.pack4(oracle.unpack4(b)) == b).all()
    q = np.random.default_rng(3).integers(0, 16, (7, 64))
    assert (oracle.unpack4(oracle.pack4(q)) == q).all()


# -- dequantization -------------------------------------------------------------

def test_e1_dequant_and_gemm(golden_dir):
    e = load(golden_dir, "e1_w4_groupwise.json")
    packed = oracle.pack4(e["codes"])
    assert packed.tolist() == e["packed"]
    s, z = bf16_bits(e["scale"]), bf16_bits(e["zero"])
    W = oracle.dequant4(packed, s, z, e["group"], BF16)
    assert W.tolist() == e["W"]
    A = bf16_bits(e["A"])
    assert oracle.gemm_w4(A, packed, s, z, e["group"], BF16).tolist() == e["C"]
    b = f16_bits(e["bias"])
    C = oracle.gemm_w4(A, packed, s, z, e["group"], BF16, bias=b, bias_dtype=FP16)
    assert C.tolist() == e["C_bias"]
    # the same numbers through fp16 activations/scales
    W16 = oracle.dequant4(packed, f16_bits(e["scale"]), f16_bits(e["zero"]), e["group"], FP16)
    assert W16.tolist() == e["W"]


def test_e1_embedding_rows(golden_dir):
    # [cpuint4] CPUInt4EmbeddingMethod.embedding: a token's row of the
    # quantized table, dequantized.  With E1's table the rows are E1's W;
    # ids outside the table give zeros (this oracle's reading).
    e = load(golden_dir, "e1_w4_groupwise.json")
    packed = np.array(e["packed"], dtype=np.uint8)
    s, z = bf16_bits(e["scale"]), bf16_bits(e["zero"])
    out = oracle.embed4([1, 0, 1, -1, 2], packed, s, z, e["group"], BF16)
    W, zero_row = e["W"], [0.0] * e["k"]
    assert out.tolist() == [W[1], W[0], W[1], zero_row, zero_row]
    # scale-only (no zeros) rows: (q - 8) * s by hand from E1's codes
    q, sc = np.array(e["codes"]), np.array(e["scale"])
    hand = (q - 8) * np.repeat(sc, e["group"], axis=1)
    assert oracle.embed4([0, 1], packed, s, None, e["group"], BF16).tolist() == hand.tolist()


def test_e2_embedding_rows(golden_dir):
    e = load(golden_dir, "e2_w8_perchannel.json")
    codes = np.array(e["codes"], dtype=np.int8)
    out = oracle.embed8([1, 1, 0, 5], codes, f16_bits(e["scale"]), -1, FP16)
    assert out.tolist() == [e["W"][1], e["W"][1], e["W"][0], [0.0] * codes.shape[1]]


def test_e2_w8_dequant_and_gemm(golden_dir):
    e = load(golden_dir, "e2_w8_perchannel.json")
    codes = np.array(e["codes"], dtype=np.int8)
    assert codes.view(np.uint8).tolist() == e["bytes"]
    s = f16_bits(e["scale"])
    assert oracle.dequant8(codes, s, -1, FP16).tolist() == e["W"]
    assert oracle.dequant8(codes, s, codes.shape[1], FP16).tolist() == e["W"]  # group = K
    C = oracle.gemm_w8(f16_bits(e["A"]), codes, s, -1, FP16)
    assert C.tolist() == e["C"]


def test_dequant_identity_grid():
    # scale 1, zero 8 turns the rule into w = q exactly
    q = np.random.default_rng(4).integers(0, 16, (8, 128))
    W = oracle.dequant4(oracle.pack4(q), bf16_bits(np.ones((8, 2))), bf16_bits(np.full((8, 2), 8.0)), 64)
    assert (W == q).all()


@pytest.mark.parametrize("j", [0, 3, 7])
def test_quantizer_extremes_identity(j):
    # scale = (max - min) / 15 and zero = min + 8 * scale put q = 0 on the
    # group minimum and q = 15 on the group maximum.  Dyadic min/max keep
    # every quantity exact in bf16.
    wmin = -1.0 + 0.25 * j
    scale = 2.0 ** -j
    wmax = wmin + 15 * scale
    zero = wmin + 8 * scale
    q = np.array([[0, 15] * 32])
    W = oracle.dequant4(oracle.pack4(q), bf16_bits([[scale]]), bf16_bits([[zero]]), 64)
    assert W[0, 0] == wmin and W[0, 1] == wmax


# -- groupwise quantizer ([cpuint4] quantize_groupwise) --------------------------

@pytest.mark.parametrize("group", [64, 128])
def test_quantize4_grid_values_recover_their_codes(group):
    # Values on a dyadic grid lo + q * step, each group holding q = 0 and
    # q = 15: scale = (hi - lo) / 15 = step and zero = lo + 8 * step exactly,
    # and every value maps back to its own q (low nibble = even k).
    rng = np.random.default_rng(group)
    n, k = 6, 4 * group
    q = rng.integers(0, 16, (n, k))
    q[:, ::group] = 0
    q[:, 1::group] = 15
    step = 2.0 ** -rng.integers(2, 7, (n, k // group))
    lo = rng.integers(-32, 33, (n, k // group)) / 8.0
    w = (np.repeat(lo, group, axis=1) + q * np.repeat(step, group, axis=1)).astype(np.float32)
    packed, scale, zero = oracle.quantize4(w, group)
    assert np.array_equal(oracle.unpack4(packed), q)
    assert np.array_equal(packed[:, 0] & 0xF, q[:, 0]) and np.array_equal(packed[:, 0] >> 4, q[:, 1])
    assert np.array_equal(scale, step.astype(np.float32))
    assert np.array_equal(zero, (lo + 8 * step).astype(np.float32))


def test_quantize4_ties_round_half_to_even():
    # lo = 0, hi = 15: step 1, so (w - lo) / scale = w exactly; halves go to
    # the even neighbour (torch's round), not up.
    w = np.zeros((1, 64), dtype=np.float32)
    w[0, 1] = 15.0
    halves = [0.5, 1.5, 2.5, 3.5, 6.5, 7.5, 8.5, 13.5, 14.5]
    w[0, 2:2 + len(halves)] = halves
    packed, scale, zero = oracle.quantize4(w, 64)
    codes = oracle.unpack4(packed)[0]
    assert scale[0, 0] == 1.0 and zero[0, 0] == 8.0
    assert codes[2:2 + len(halves)].tolist() == [0, 2, 2, 4, 6, 8, 8, 14, 14]


def test_quantize4_constant_group():
    # hi = lo: the range is clamped to 1e-9 before the division by 15; every
    # code is 0 and the dequantized value is lo up to the zero's rounding.
    w = np.full((2, 128), -0.75, dtype=np.float32)
    packed, scale, zero = oracle.quantize4(w, 64)
    assert (oracle.unpack4(packed) == 0).all()
    assert (scale == np.float32(np.float32(1e-9) / np.float32(15.0))).all()
    assert (zero == np.float32(np.float32(-0.75) + np.float32(8.0) * scale)).all()


@pytest.mark.parametrize("group", [64, 128])
def test_quantize4_error_within_half_a_step(group):
    # Nearest point of the grid lo + q * scale: the reconstruction
    # (q - 8) * scale + zero is within scale / 2 of w (plus fp32 rounding of
    # the quotient, the zero and the difference), and each group's extremes
    # get codes 0 and 15.
    rng = np.random.default_rng(9 + group)
    n, k = 64, 1024
    w = (rng.standard_normal((n, k)) * rng.uniform(0.01, 2.0, (n, 1))).astype(np.float32)
    packed, scale, zero = oracle.quantize4(w, group)
    q = oracle.unpack4(packed)
    s = np.repeat(scale.astype(np.float64), group, axis=1)
    z = np.repeat(zero.astype(np.float64), group, axis=1)
    rec = (q - 8) * s + z
    wd = w.astype(np.float64)
    slack = 2.0 ** -21 * (np.abs(wd) + np.abs(z) + 16 * s)
    assert (np.abs(rec - wd) <= 0.5 * s + slack).all()
    g = w.reshape(n, k // group, group)
    qg_ = q.reshape(n, k // group, group)
    rows, grp = np.indices(g.shape[:2])
    assert (qg_[rows, grp, g.argmin(axis=2)] == 0).all()
    assert (qg_[rows, grp, g.argmax(axis=2)] == 15).all()


def test_group_indexing_closed_form():
    # constant code c and A = 1: C[n] = sum_g group * ((c - 8) * s[n, g] + z[n, g])
    rng = np.random.default_rng(5)
    n, k, g, c = 5, 512, 64, 11
    s = (rng.integers(1, 64, (n, k // g)) / 64.0).astype(np.float32)
    z = (rng.integers(-32, 33, (n, k // g)) / 64.0).astype(np.float32)
    packed = oracle.pack4(np.full((n, k), c))
    C = oracle.gemm_w4(bf16_bits(np.ones((1, k))), packed, bf16_bits(s), bf16_bits(z), g)
    expect = (g * ((c - 8) * s.astype(np.float64) + z)).sum(axis=1)
    assert np.array_equal(C[0], expect)


@pytest.mark.parametrize("group", [-1, 1024])
def test_per_column_closed_form(group):
    # One scale and zero per channel (group -1, or k itself): with a constant
    # code c and A = 1, C[n] = k * ((c - 8) * s[n] + z[n]), exact in double.
    rng = np.random.default_rng(15)
    n, k, c = 6, 1024, 3
    s = (rng.integers(1, 64, (n,)) / 64.0).astype(np.float32)
    z = (rng.integers(-32, 33, (n,)) / 64.0).astype(np.float32)
    packed = oracle.pack4(np.full((n, k), c))
    C = oracle.gemm_w4(bf16_bits(np.ones((1, k))), packed, bf16_bits(s), bf16_bits(z), group)
    assert np.array_equal(C[0], k * ((c - 8) * s.astype(np.float64) + z))
    W = oracle.dequant4(packed, bf16_bits(s), bf16_bits(z), group)
    assert np.array_equal(W, np.repeat(((c - 8) * s + z)[:, None], k, axis=1).astype(np.float32))


def test_scale_only_closed_forms():
    # No zero points: w = (q - 8) * s.  Scale 1 turns every code into q - 8;
    # a constant code c with A = 1 sums to sum_g g * (c - 8) * s[n, g].
    q = np.random.default_rng(16).integers(0, 16, (8, 256))
    W = oracle.dequant4(oracle.pack4(q), bf16_bits(np.ones((8, 4))), None, 64)
    assert (W == q - 8).all()
    rng = np.random.default_rng(17)
    n, k, g, c = 5, 512, 128, 13
    s = (rng.integers(1, 64, (n, k // g)) / 64.0).astype(np.float32)
    C = oracle.gemm_w4(bf16_bits(np.ones((1, k))), oracle.pack4(np.full((n, k), c)), bf16_bits(s),
                       None, g)
    assert np.array_equal(C[0], (g * (c - 8) * s.astype(np.float64)).sum(axis=1))
    # per-column and scale-only together
    s1 = (rng.integers(1, 64, (n,)) / 64.0).astype(np.float32)
    C1 = oracle.gemm_w4(bf16_bits(np.ones((1, k))), oracle.pack4(np.full((n, k), c)), bf16_bits(s1),
                        None, -1)
    assert np.array_equal(C1[0], k * (c - 8) * s1.astype(np.float64))


def test_dequant_rounds_once_in_fp32():
    # (q - 8) * s is exact in fp32; only the add of the zero rounds, to nearest even.
    rng = np.random.default_rng(6)
    n, k, g = 64, 256, 64
    p = si.w4_problem(1, n, k, g)
    W = oracle.dequant4(p.packed, p.scale, p.zero, g)
    q = oracle.unpack4(p.packed).astype(np.float64)
    s = np.repeat(torch.from_numpy(p.scale.view(np.int16).copy()).view(torch.bfloat16).double().numpy(), g, axis=1)
    z = np.repeat(torch.from_numpy(p.zero.view(np.int16).copy()).view(torch.bfloat16).double().numpy(), g, axis=1)
    exact = (q - 8.0) * s + z                  # exact in double
    assert np.array_equal(W, exact.astype(np.float32))   # numpy's cast is RNE
    del rng


# -- GEMM brute force against a library matmul -----------------------------------

@pytest.mark.parametrize("m,n,k,g", [(1, 16, 64, 64), (3, 40, 128, 64), (7, 64, 256, 128), (5, 33, 192, 64)])
@pytest.mark.parametrize("dtype", [BF16, FP16])
def test_w4_gemm_vs_numpy_matmul(m, n, k, g, dtype):
    p = si.w4_problem(m, n, k, g, tag="pin", dtype=dtype, bias_dtype=FP16)
    W = oracle.dequant4(p.packed, p.scale, p.zero, g, dtype).astype(np.float64)
    conv = oracle.bf16_to_f32 if dtype == BF16 else oracle.f16_to_f32
    A = conv(p.A).astype(np.float64)
    bias = oracle.f16_to_f32(p.bias).astype(np.float64)
    ref = A @ W.T + bias
    C = oracle.gemm_w4(p.A, p.packed, p.scale, p.zero, g, dtype, p.bias, FP16)
    np.testing.assert_allclose(C, ref, rtol=1e-12, atol=1e-12)
    rows = np.array([0, m - 1, m // 2]); cols = np.array([n - 1, 0, n // 3])
    at = oracle.gemm_w4_at(p.A, p.packed, p.scale, p.zero, g, rows, cols, dtype, p.bias, FP16)
    np.testing.assert_allclose(at, ref[rows, cols], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("m,n,k", [(1, 16, 64), (4, 24, 96), (9, 8, 256)])
def test_w8_gemm_vs_numpy_matmul(m, n, k):
    p = si.w8_problem(m, n, k, -1, tag="pin", bias_dtype=FP16)
    W = oracle.dequant8(p.codes, p.scale, -1, FP16).astype(np.float64)
    A = oracle.f16_to_f32(p.A).astype(np.float64)
    ref = A @ W.T + oracle.f16_to_f32(p.bias)
    C = oracle.gemm_w8(p.A, p.codes, p.scale, -1, FP16, p.bias, FP16)
    np.testing.assert_allclose(C, ref, rtol=1e-12, atol=1e-12)
    # signed codes: the weight is the code times the scale, sign included
    s = oracle.f16_to_f32(p.scale).astype(np.float64)
    assert np.array_equal(W, p.codes.astype(np.float64) * s[:, None])


# -- W8A8 ([acext] 1.2.2, 1.3.4) ----------------------------------------------------

def test_w8a8_worked_example():
    # Row [1, -2, 3] against weight rows [4, 5, -6] and [127, -128, 1]: the
    # integer sums are 4 - 10 - 18 = -24 and 127 + 256 + 3 = 386; with the
    # per-tensor activation scale 2 and per-channel scales [0.5, 0.25]:
    # C = [-24, 193].
    acc, C = oracle.gemm_w8a8(np.array([[1, -2, 3]], np.int8),
                              np.array([[4, 5, -6], [127, -128, 1]], np.int8), [2.0], [0.5, 0.25])
    assert acc.tolist() == [[-24, 386]] and C.tolist() == [[-24.0, 193.0]]


@pytest.mark.parametrize("per_token,per_channel", [(0, 0), (0, 1), (1, 0), (1, 1)])
def test_w8a8_vs_numpy_integer_matmul(per_token, per_channel):
    # The four QuantMode variants: the exact int64 product from numpy, times
    # the row and column scales (one value each when per tensor).
    rng = np.random.default_rng(per_token * 2 + per_channel)
    m, n, k = 7, 24, 320
    A = rng.integers(-128, 128, (m, k)).astype(np.int8)
    B = rng.integers(-128, 128, (n, k)).astype(np.int8)
    ar = rng.uniform(0.001, 0.1, m if per_token else 1).astype(np.float32)
    ac = rng.uniform(0.001, 0.1, n if per_channel else 1).astype(np.float32)
    acc, C = oracle.gemm_w8a8(A, B, ar, ac)
    ref_acc = A.astype(np.int64) @ B.astype(np.int64).T
    assert np.array_equal(acc, ref_acc)
    scale = np.outer(np.broadcast_to(ar.astype(np.float64), (m,)),
                     np.broadcast_to(ac.astype(np.float64), (n,)))
    np.testing.assert_allclose(C, ref_acc * scale, rtol=1e-15)


def test_w8a8_extremes():
    # -128 * -128 over k = 4096 is 2^26, beyond int32's fp32-exact range but
    # exact in the int64 sum.
    k = 4096
    acc, C = oracle.gemm_w8a8(np.full((1, k), -128, np.int8), np.full((2, k), -128, np.int8),
                              [1.0], [1.0])
    assert (acc == 16384 * k).all() and (C == 16384.0 * k).all()


def test_w4_exact_inputs_are_exact():
    p = si.w4_exact_problem(3, 32, 256, 64, seed=7, bias_dtype=FP16)
    C = oracle.gemm_w4(p.A, p.packed, p.scale, p.zero, 64, BF16, p.bias, FP16)
    assert np.array_equal(C * 4, np.round(C * 4))     # multiples of 1/4
    assert np.abs(C).max() < 2 ** 17


# -- MoE ---------------------------------------------------------------------

def test_route_one_hot_and_ties():
    lg = np.zeros((3, 8), np.float32)
    lg[0, 5] = 4.0; lg[0, 2] = 3.0
    lg[1, :] = 1.0                                   # all tied: lowest ids first
    lg[2, 7] = 2.0; lg[2, 1] = 2.0; lg[2, 0] = -1.0
    ids, w = oracle.moe_route(lg, 2)
    assert ids.tolist() == [[5, 2], [0, 1], [1, 7]]
    np.testing.assert_allclose(w[0], [np.exp(1) / (np.exp(1) + 1), 1 / (np.exp(1) + 1)], rtol=1e-15)
    np.testing.assert_allclose(w[1], [0.5, 0.5], rtol=0)
    np.testing.assert_allclose(w[2], [0.5, 0.5], rtol=0)


def test_route_weights_are_renormalised_softmax():
    lg = np.random.default_rng(8).standard_normal((50, 16)).astype(np.float32)
    ids, w = oracle.moe_route(lg, 4)
    np.testing.assert_allclose(w.sum(1), 1.0, rtol=1e-14)
    sm = torch.softmax(torch.from_numpy(lg).double(), dim=1).numpy()
    top = np.take_along_axis(sm, ids.astype(np.int64), 1)
    np.testing.assert_allclose(w, top / top.sum(1, keepdims=True), rtol=1e-12)
    assert (np.diff(np.take_along_axis(lg, ids.astype(np.int64), 1), axis=1) <= 0).all()
    ids1, w1 = oracle.moe_route(lg, 1)
    assert (w1 == 1.0).all() and (ids1[:, 0] == lg.argmax(1)).all()


def _dense_swiglu(xf, W1, W2, inter):
    h = xf @ W1.T
    gate, up = h[:, :inter], h[:, inter:]
    a = gate / (1.0 + np.exp(-gate)) * up
    return a @ W2.T


def _conv(bits, dtype):
    return (oracle.bf16_to_f32(bits) if dtype == BF16 else oracle.f16_to_f32(bits)).astype(np.float64)


def test_moe_identical_experts_equal_dense_ffn():
    p = si.moe_problem(6, 64, 64, 4, 2, group=64, tag="pin-moe")
    for arr in (p.w1, p.s1, p.z1, p.w2, p.s2, p.z2):
        arr[1:] = arr[0]
    out, _, _ = oracle.moe(p.x, p.logits, p.w1, p.s1, p.z1, p.w2, p.s2, p.z2, 2, 64)
    W1 = oracle.dequant4(p.w1[0], p.s1[0], p.z1[0], 64).astype(np.float64)
    W2 = oracle.dequant4(p.w2[0], p.s2[0], p.z2[0], 64).astype(np.float64)
    ref = _dense_swiglu(_conv(p.x, BF16), W1, W2, 64)
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-10)


def test_moe_brute_force_tiny():
    p = si.moe_problem(4, 64, 64, 4, 2, group=64, tag="pin-moe2")
    out, ids, w = oracle.moe(p.x, p.logits, p.w1, p.s1, p.z1, p.w2, p.s2, p.z2, 2, 64)
    xf = _conv(p.x, BF16)
    ref = np.zeros_like(out)
    for e in range(4):
        W1 = oracle.dequant4(p.w1[e], p.s1[e], p.z1[e], 64).astype(np.float64)
        W2 = oracle.dequant4(p.w2[e], p.s2[e], p.z2[e], 64).astype(np.float64)
        ye = _dense_swiglu(xf, W1, W2, 64)
        for t in range(4):
            for j in range(2):
                if ids[t, j] == e:
                    ref[t] += w[t, j] * ye[t]
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-10)


def test_moe_expert_permutation_invariance():
    p = si.moe_problem(5, 64, 64, 4, 2, group=64, tag="pin-moe3")
    out, _, _ = oracle.moe(p.x, p.logits, p.w1, p.s1, p.z1, p.w2, p.s2, p.z2, 2, 64)
    perm = np.array([2, 0, 3, 1])
    out2, _, _ = oracle.moe(p.x, p.logits[:, perm], p.w1[perm], p.s1[perm], p.z1[perm],
                            p.w2[perm], p.s2[perm], p.z2[perm], 2, 64)
    np.testing.assert_allclose(out, out2, rtol=1e-13, atol=1e-13)


def test_moe_token_subset_matches_full():
    p = si.moe_problem(6, 64, 128, 4, 3, group=64, tag="pin-moe4")
    full, _, _ = oracle.moe(p.x, p.logits, p.w1, p.s1, p.z1, p.w2, p.s2, p.z2, 3, 64)
    part, _, _ = oracle.moe(p.x, p.logits, p.w1, p.s1, p.z1, p.w2, p.s2, p.z2, 3, 64, tokens=[4, 1])
    np.testing.assert_array_equal(part, full[[4, 1]])


# -- MoE extras: selection logits with bias, normalization mode, finished rows,
# fc1 / fc2 expert biases ([acext] 1.2.3 runMoe) ---------------------------------

def test_moe_route_selection_bias_hand_worked():
    # Gating logits l = [0, 1, 2, 3]; the biased selection logits
    # [5, 1, 2, 0] choose experts 0 and 2; the weights come from l:
    # exp(0) / (exp(0) + exp(2)) and exp(2) / (exp(0) + exp(2)).
    l = np.array([[0.0, 1.0, 2.0, 3.0]], np.float32)
    sl = np.array([[5.0, 1.0, 2.0, 0.0]], np.float32)
    ids, w = oracle.moe_route(l, 2, sel_logits=sl)
    assert ids.tolist() == [[0, 2]]
    e2 = np.exp(2.0)
    np.testing.assert_allclose(w[0], [1 / (1 + e2), e2 / (1 + e2)], rtol=1e-15)
    ids, w = oracle.moe_route(l, 2)                    # without the bias: 3, 2
    assert ids.tolist() == [[3, 2]]


def test_moe_route_no_renormalization_is_softmax_probability():
    # Logits log(1..4): the softmax over all four is [0.1, 0.2, 0.3, 0.4];
    # without renormalization the top-2 keep their probabilities 0.4, 0.3.
    l = np.log(np.array([[1.0, 2.0, 3.0, 4.0]])).astype(np.float32)
    ids, w = oracle.moe_route(l, 2, renormalize=False)
    assert ids.tolist() == [[3, 2]]
    np.testing.assert_allclose(w[0], [0.4, 0.3], rtol=1e-6)
    _, w1 = oracle.moe_route(l, 1, renormalize=True)
    assert w1.tolist() == [[1.0]]


def test_moe_finished_rows_take_no_expert():
    p = si.moe_problem(5, 64, 64, 4, 2, group=64, tag="pin-moe5")
    fin = np.array([0, 1, 0, 0, 1], np.uint8)
    out, ids, w = oracle.moe(p.x, p.logits, p.w1, p.s1, p.z1, p.w2, p.s2, p.z2, 2, 64, finished=fin)
    assert (ids[fin == 1] == -1).all() and (w[fin == 1] == 0).all()
    assert (out[fin == 1] == 0).all()
    full, ids0, _ = oracle.moe(p.x, p.logits, p.w1, p.s1, p.z1, p.w2, p.s2, p.z2, 2, 64)
    np.testing.assert_array_equal(out[fin == 0], full[fin == 0])
    np.testing.assert_array_equal(ids[fin == 0], ids0[fin == 0])


def _dense_swiglu_bias(xf, W1, b1, W2, b2, inter):
    h = xf @ W1.T + b1
    gate, up = h[:, :inter], h[:, inter:]
    a = gate / (1.0 + np.exp(-gate)) * up
    return a @ W2.T + b2


@pytest.mark.parametrize("renormalize", [True, False])
def test_moe_identical_experts_with_biases_equal_dense_ffn(renormalize):
    # Every expert the same (weights and biases): with renormalized weights
    # the output is the dense biased SwiGLU FFN; without, that FFN times the
    # sum of the selected probabilities.
    p = si.moe_problem(6, 64, 64, 4, 2, group=64, tag="pin-moe6")
    b1, b2, _, _ = si.moe_extras(p)
    for arr in (p.w1, p.s1, p.z1, p.w2, p.s2, p.z2, b1, b2):
        arr[1:] = arr[0]
    out, _, w = oracle.moe(p.x, p.logits, p.w1, p.s1, p.z1, p.w2, p.s2, p.z2, 2, 64, b1=b1, b2=b2,
                           renormalize=renormalize)
    W1 = oracle.dequant4(p.w1[0], p.s1[0], p.z1[0], 64).astype(np.float64)
    W2 = oracle.dequant4(p.w2[0], p.s2[0], p.z2[0], 64).astype(np.float64)
    ref = _dense_swiglu_bias(_conv(p.x, BF16), W1, _conv(b1[0], BF16), W2, _conv(b2[0], BF16), 64)
    np.testing.assert_allclose(out, ref * w.sum(axis=1, keepdims=True), rtol=1e-10, atol=1e-10)
    if renormalize:
        np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=1e-15)


# -- int8 with group scales (scale [n, k/g]) ------------------------------------------

@pytest.mark.parametrize("dtype", [FP16, BF16])
def test_e3_w8_groupwise_dequant_and_gemm(golden_dir, dtype):
    # Two K-groups with distinct scales per row: the [n, k/g] scale layout
    # gives E3's W and C; reading the scales as [k/g, n] would give the
    # fixture's W_if_scales_transposed instead.
    e = load(golden_dir, "e3_w8_groupwise.json")
    codes = np.array(e["codes"], dtype=np.int8)
    bits = f16_bits if dtype == FP16 else bf16_bits
    s = bits(e["scale"])
    W = oracle.dequant8(codes, s, e["group"], dtype)
    assert W.tolist() == e["W"] and W.tolist() != e["W_if_scales_transposed"]
    A = bits(e["A"])
    assert oracle.gemm_w8(A, codes, s, e["group"], dtype).tolist() == e["C"]
    Cb = oracle.gemm_w8(A, codes, s, e["group"], dtype, bits(e["bias"]), dtype)
    assert Cb.tolist() == e["C_bias"]
    at = oracle.gemm_w8_at(A, codes, s, [0, 0], [1, 0], e["group"], dtype, bits(e["bias"]), dtype)
    assert at.tolist() == [e["C_bias"][0][1], e["C_bias"][0][0]]


@pytest.mark.parametrize("g", [64, 128])
def test_w8_group_closed_form(g):
    # constant code c and A = 1: C[n] = sum_groups g * c * s[n, group]
    rng = np.random.default_rng(31 + g)
    n, k, c = 6, 1024, -37
    s = (rng.integers(1, 64, (n, k // g)) / 1024.0).astype(np.float32)
    codes = np.full((n, k), c, np.int8)
    C = oracle.gemm_w8(f16_bits(np.ones((1, k))), codes, f16_bits(s), g, FP16)
    assert np.array_equal(C[0], (g * c * s.astype(np.float64)).sum(axis=1))
    W = oracle.dequant8(codes, f16_bits(s), g, FP16)
    assert np.array_equal(W, c * np.repeat(s, g, axis=1))


@pytest.mark.parametrize("g", [-1, 64, 128])
@pytest.mark.parametrize("with_bias", [False, True])
def test_w8_gemm_at_vs_numpy(g, with_bias):
    # The sampled evaluation (used at full workload sizes) against numpy's
    # fp64 matmul of the dequantized weight, at chosen (row, col) pairs
    # including the corners.
    m, n, k = 6, 48, 384
    p = si.w8_problem(m, n, k, g, tag="pin-at", bias_dtype=FP16 if with_bias else 0)
    W = oracle.dequant8(p.codes, p.scale, g, FP16).astype(np.float64)
    ref = oracle.f16_to_f32(p.A).astype(np.float64) @ W.T
    if with_bias:
        ref = ref + oracle.f16_to_f32(p.bias)
    rows = np.array([0, m - 1, 3, 0, m - 1, 2])
    cols = np.array([0, n - 1, 17, n - 1, 0, 40])
    at = oracle.gemm_w8_at(p.A, p.codes, p.scale, rows, cols, g, FP16,
                           p.bias if with_bias else None, FP16 if with_bias else 0)
    np.testing.assert_allclose(at, ref[rows, cols], rtol=1e-12, atol=1e-12)


# -- fp32-accumulating variant (the timed CPU baseline) ------------------------------

@pytest.mark.parametrize("m,n,k,g,bias", [(4, 128, 256, 64, False), (1, 2048, 2048, 64, False),
                                          (3, 256, 2048, 128, True)])
def test_w4_f32acc_agrees_with_double(m, n, k, g, bias):
    # Same sums carried in fp32: they must agree with the double definition
    # to within 1e-4 of the largest output (fp32 rounding of a K-term sum).
    p = si.w4_problem(m, n, k, g, tag="f32acc", bias_dtype=FP16 if bias else 0)
    kw = dict(bias=p.bias, bias_dtype=FP16) if bias else {}
    ref = oracle.gemm_w4(p.A, p.packed, p.scale, p.zero, g, BF16, **kw)
    got = oracle.gemm_w4_f32acc(p.A, p.packed, p.scale, p.zero, g, BF16, **kw)
    assert got.dtype == np.float32
    assert np.abs(got - ref).max() <= 1e-4 * np.abs(ref).max()
    assert not np.array_equal(got.astype(np.float64), ref)   # really a different sum


@pytest.mark.parametrize("g", [-1, 128])
def test_w8_f32acc_agrees_with_double(g):
    p = si.w8_problem(2, 512, 3584, g, tag="f32acc8")
    ref = oracle.gemm_w8(p.A, p.codes, p.scale, g, FP16)
    got = oracle.gemm_w8_f32acc(p.A, p.codes, p.scale, g, FP16)
    assert np.abs(got - ref).max() <= 1e-4 * np.abs(ref).max()


def test_f32acc_exact_inputs_equal_double():
    # Integer/dyadic inputs: every partial sum is exact in fp32, so the two
    # accumulations give identical results.
    p = si.w4_exact_problem(3, 64, 512, 64, seed=11, bias_dtype=FP16)
    ref = oracle.gemm_w4(p.A, p.packed, p.scale, p.zero, 64, BF16, p.bias, FP16)
    got = oracle.gemm_w4_f32acc(p.A, p.packed, p.scale, p.zero, 64, BF16, p.bias, FP16)
    assert np.array_equal(got.astype(np.float64), ref)


# -- routing with -inf selection logits ------------------------------------------------

def test_route_neg_inf_selection_logits_give_distinct_ids():
    # Selection logits [-inf, 2, -inf, 1, -inf] with top-4: experts 1 and 3
    # first, then the untaken -inf experts in index order, 0 then 2 (ties to
    # the lower index); an expert is never chosen twice.  Weights come from
    # the gating logits l = [0, 1, 2, 3, 4] over the chosen set {1, 3, 0, 2}.
    ninf = -np.inf
    sl = np.array([[ninf, 2.0, ninf, 1.0, ninf]], np.float32)
    l = np.array([[0.0, 1.0, 2.0, 3.0, 4.0]], np.float32)
    ids, w = oracle.moe_route(l, 4, sel_logits=sl)
    assert ids.tolist() == [[1, 3, 0, 2]]
    e = np.exp(np.array([1.0, 3.0, 0.0, 2.0]))
    np.testing.assert_allclose(w[0], e / e.sum(), rtol=1e-15)
    # all selection logits -inf: index order
    ids, _ = oracle.moe_route(l, 5, sel_logits=np.full((1, 5), ninf, np.float32))
    assert ids.tolist() == [[0, 1, 2, 3, 4]]
