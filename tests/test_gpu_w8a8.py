"""GPU parity of the W8A8 GEMM (int8 activations x int8 weights, fp32 row
and column scales; acext User Guide (v1.7), 1.2.2 and 1.3.4) against the
oracle's exact int64 sums.

Integer work is checked bit for bit: with unit or power-of-two scales and
|sum| below 2^24 the fp32 output is the exact sum times the scales.  Random
scales are checked to the output dtype's tolerance (fp32 output: the three
roundings of float(sum) * row * col, elementwise)."""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
import weight_only_quantized_w8a16_amd as qg
from helpers import rel_err

pytestmark = pytest.mark.gpu

TILES = ["T256", "T256N", "T128", "T64"]
OUT = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}
TOL = {"fp16": 3e-3, "bf16": 1e-2}


def run(p, out="fp32", workspace=True):
    dev = "cuda"
    A, B = torch.from_numpy(p.A).to(dev), torch.from_numpy(p.B).to(dev)
    ar, ac = torch.from_numpy(p.alpha_row).to(dev), torch.from_numpy(p.alpha_col).to(dev)
    ws = None
    if not workspace:
        ws = torch.empty(0, dtype=torch.uint8, device=dev)   # no room: unsplit
    C = qg.gemm_w8a8(A, B, ar, ac, out_dtype=OUT[out], workspace=ws)
    torch.cuda.synchronize()
    return C.float().cpu().numpy().astype(np.float64)


def ref(p):
    acc, C = oracle.gemm_w8a8(p.A, p.B, p.alpha_row, p.alpha_col)
    return acc, C


# -- exact: unit scales, fp32 output, |sum| < 2^24 ---------------------------------

@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("m,n,k", [(1, 128, 128), (5, 144, 256), (70, 272, 384), (200, 400, 512),
                                   (300, 528, 1024)])
def test_w8a8_integer_sums_bit_exact(tile, m, n, k):
    # Several tiles in each direction, ragged M and N tails (n % 128 != 0).
    qg.set_override(w8a8_tile=tile)
    p = si.w8a8_problem(m, n, k, False, False, scales=[1.0])
    acc, _ = ref(p)
    assert np.abs(acc).max() < 2 ** 24
    C = run(p)
    assert np.array_equal(C, acc.astype(np.float64))


@pytest.mark.parametrize("m,n,k", [(1, 16, 128), (1, 528, 384), (5, 144, 1024), (16, 8192, 896), (1, 8192, 768),
                                   (9, 3584, 3584), (16, 18944, 1024),
                                   # one tile per workgroup, 17 and 15 chunks over up to 16 waves
                                   (2, 48, 2176), (3, 32, 1920),
                                   # from 8 rows the weight chunks go through LDS
                                   (8, 8192, 1280), (12, 64, 384), (8, 48, 2176)])
def test_w8a8_decode_kernel_bit_exact(m, n, k):
    # m <= 16 runs the streaming decode kernel (one or two 16-channel tiles
    # per workgroup, waves over 128- or 256-k chunks; from 8 rows each chunk
    # staged through the wave's LDS area); unit and power-of-two scales keep
    # the fp32 output exact.
    p = si.w8a8_problem(m, n, k, False, False, scales=[1.0])
    acc, _ = ref(p)
    if np.abs(acc).max() < 2 ** 24:
        assert np.array_equal(run(p), acc.astype(np.float64))
    for pt, pc in ((0, 1), (1, 0), (1, 1)):
        p = si.w8a8_problem(m, n, k, bool(pt), bool(pc), scales=[0.25, 0.5, 1.0, 2.0],
                            code_range=(-64, 64))
        _, Cref = ref(p)
        if np.abs(Cref).max() < 2 ** 24 / 8:
            assert np.array_equal(run(p), Cref)


@pytest.mark.parametrize("m,n,k", [(64, 3584, 3584), (32, 3584, 1024), (40, 1040, 2048)])
def test_w8a8_split_k_equals_unsplit_bitwise(m, n, k):
    # Problems with few 64 x 128 tiles are split along K into int32 partials;
    # integer sums are exact in any order, so split and unsplit agree bit for
    # bit.
    qg.set_override(w8a8_tile="T64")
    assert qg.w8a8_workspace_size(m, n, k) > 0
    p = si.w8a8_problem(m, n, k, True, True)
    assert np.array_equal(run(p, "fp32", True), run(p, "fp32", False))
    p1 = si.w8a8_problem(m, n, min(k, 1024), False, False, scales=[1.0])
    acc, _ = ref(p1)
    assert np.array_equal(run(p1, "fp32", True), acc.astype(np.float64))


@pytest.mark.parametrize("per_token,per_channel", [(0, 0), (0, 1), (1, 0), (1, 1)])
@pytest.mark.parametrize("tile", ["T256", "T64"])
def test_w8a8_power_of_two_scales_bit_exact(per_token, per_channel, tile):
    # Power-of-two scales keep every product exact: C == sum * row * col.
    qg.set_override(w8a8_tile=tile)
    p = si.w8a8_problem(260, 400, 512, bool(per_token), bool(per_channel),
                        scales=[0.25, 0.5, 1.0, 2.0, 0.125])
    _, Cref = ref(p)
    assert np.array_equal(run(p), Cref)


def test_w8a8_extreme_codes_at_largest_k():
    # -128 x -128 over the largest accepted k: the sum 2^14 k stays below 2^31.
    k = 130944
    p = si.w8a8_problem(2, 16, k, False, False, code_range=(-128, -128), scales=[1.0])
    acc, Cref = ref(p)
    assert acc.max() == 16384 * k < 2 ** 31
    C = run(p)
    assert np.array_equal(C, np.float32(Cref).astype(np.float64))


# -- random scales, every mode and output dtype -------------------------------------

@pytest.mark.parametrize("out", ["fp32", "fp16", "bf16"])
@pytest.mark.parametrize("per_token,per_channel", [(0, 0), (0, 1), (1, 0), (1, 1)])
@pytest.mark.parametrize("m,n,k", [(4, 256, 512), (96, 384, 768), (520, 512, 1024)])
def test_w8a8_random_scales(per_token, per_channel, out, m, n, k):
    p = si.w8a8_problem(m, n, k, bool(per_token), bool(per_channel))
    _, Cref = ref(p)
    C = run(p, out)
    if out == "fp32":
        # float(sum) and the two products each round once (<= 2^-24 relative).
        assert np.all(np.abs(C - Cref) <= 4e-7 * np.abs(Cref))
    else:
        assert rel_err(C, Cref) <= TOL[out]


def test_w8a8_leading_dims_and_empty():
    p = si.w8a8_problem(6, 128, 256, True, True)
    _, Cref = ref(p)
    dev = "cuda"
    A = torch.from_numpy(p.A).to(dev).reshape(2, 3, 256)
    C = qg.gemm_w8a8(A, torch.from_numpy(p.B).to(dev), torch.from_numpy(p.alpha_row).to(dev),
                     torch.from_numpy(p.alpha_col).to(dev), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert C.shape == (2, 3, 128)
    assert np.all(np.abs(C.reshape(6, 128).cpu().numpy() - Cref) <= 4e-7 * np.abs(Cref))
    E = qg.gemm_w8a8(torch.empty((0, 256), dtype=torch.int8, device=dev),
                     torch.from_numpy(p.B).to(dev), torch.ones(1, device=dev),
                     torch.ones(1, device=dev))
    assert E.shape == (0, 128)


# -- the SmoothQuant-sized workload (K = 3584, N in {3584, 18944}), sampled ----------

@pytest.mark.parametrize("m", [1, 16, 128, 1024, 4096])
@pytest.mark.parametrize("n", [3584, 18944])
def test_w8a8_full_size_sampled(m, n):
    # Full-size launch as the benchmark runs it (auto tile and split); the
    # oracle computes the sampled rows x columns sub-problem.
    k = 3584
    p = si.w8a8_problem(m, n, k, True, True, tag="w8a8-bench")
    C = run(p, "fp16")
    rng = np.random.default_rng(m + n)
    rows = np.unique(np.concatenate([[0, m - 1], rng.integers(0, m, 6)]))
    cols = np.unique(np.concatenate([[0, n - 1], rng.integers(0, n, 24)]))
    _, Cs = oracle.gemm_w8a8(p.A[rows], p.B[cols], p.alpha_row[rows], p.alpha_col[cols])
    assert rel_err(C[np.ix_(rows, cols)], Cs) <= TOL["fp16"]
