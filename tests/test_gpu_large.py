"""Maximum sizes: operands past 2 GiB.

The direct-load prefill tiles address their operands through buffer
resources with 32-bit offsets, so the library hands a problem whose packed
weights or activations reach 2^31 bytes to the generic tile of the same
width (64-bit addressing); the decode kernels use 64-bit offsets throughout.
These tests run such problems on both paths, from the same device weights,
and compare sampled outputs with the oracle (evaluated one by one)."""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
import weight_only_quantized_w8a16_amd as qg
from helpers import BF16, FP16, TOL, to_dev

pytestmark = pytest.mark.gpu

K = 32768


def _pairs(m, n, seed, count=96):
    rng = np.random.default_rng(seed)
    rows = np.concatenate([[0, m - 1], rng.integers(0, m, count)])
    cols = np.concatenate([[0, n - 1], rng.integers(0, n, count)])
    return rows, cols


def _check(C, ref, rows, cols, dtype, what):
    got = C[torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()].float().cpu().numpy()
    err = np.abs(got - ref).max() / np.abs(ref).max()
    assert err <= TOL[dtype], (what, err)


def test_w4_weights_past_2gib():
    # N * K / 2 = 2^31 bytes of packed codes (a 131072-row table at K = 32768)
    n, g = 131072, 64
    p = si.w4_problem(300, n, K, g, tag="large-w4")
    assert p.packed.nbytes >= 2 ** 31
    tiled = qg.repack_w4(to_dev(p.packed))
    S, Z = to_dev(p.scale, BF16), to_dev(p.zero, BF16)
    A = to_dev(p.A, BF16)
    C = qg.gemm_w4a16(A, tiled, S, Z, None, g)             # prefill (generic tile)
    C1 = qg.gemm_w4a16(A[:1], tiled, S, Z, None, g)        # decode
    torch.cuda.synchronize()
    rows, cols = _pairs(300, n, 1)
    _check(C, oracle.gemm_w4_at(p.A, p.packed, p.scale, p.zero, g, rows, cols, BF16),
           rows, cols, BF16, "prefill")
    zero_rows = np.zeros_like(cols)
    _check(C1, oracle.gemm_w4_at(p.A, p.packed, p.scale, p.zero, g, zero_rows, cols, BF16),
           zero_rows, cols, BF16, "decode")
    del tiled, S, Z, A, C, C1
    torch.cuda.empty_cache()


def test_w8_weights_past_2gib():
    # N * K = 2^31 bytes of int8 codes, one scale per channel
    n = 65536
    p = si.w8_problem(300, n, K, tag="large-w8", dtype=FP16)
    assert p.codes.nbytes >= 2 ** 31
    tiled = qg.repack_w8(to_dev(p.codes))
    S, A = to_dev(p.scale, FP16), to_dev(p.A, FP16)
    C = qg.gemm_w8a16(A, tiled, S, None, -1)
    C1 = qg.gemm_w8a16(A[:1], tiled, S, None, -1)
    torch.cuda.synchronize()
    rows, cols = _pairs(300, n, 2)
    _check(C, oracle.gemm_w8_at(p.A, p.codes, p.scale, rows, cols, -1, FP16),
           rows, cols, FP16, "prefill")
    zero_rows = np.zeros_like(cols)
    _check(C1, oracle.gemm_w8_at(p.A, p.codes, p.scale, zero_rows, cols, -1, FP16),
           zero_rows, cols, FP16, "decode")
    del tiled, S, A, C, C1
    torch.cuda.empty_cache()


def test_w4_activations_past_2gib():
    # M * K * 2 bytes of bf16 activations past 2^31 (65552 rows, a ragged
    # last 256-row tile), groups of 128
    m, n, g = 65552, 256, 128
    p = si.w4_problem(m, n, K, g, tag="large-a", bias_dtype=FP16)
    assert p.A.nbytes >= 2 ** 31
    tiled = qg.repack_w4(to_dev(p.packed))
    C = qg.gemm_w4a16(to_dev(p.A, BF16), tiled, to_dev(p.scale, BF16), to_dev(p.zero, BF16),
                      to_dev(p.bias, FP16), g)
    torch.cuda.synchronize()
    rows, cols = _pairs(m, n, 3)
    rows = np.concatenate([rows, [m - 16, 65535, 65536]])
    cols = np.concatenate([cols, [5, 250, 128]])
    _check(C, oracle.gemm_w4_at(p.A, p.packed, p.scale, p.zero, g, rows, cols, BF16, p.bias, FP16),
           rows, cols, BF16, "prefill")
    del tiled, C
    torch.cuda.empty_cache()


@pytest.mark.parametrize("m", [32767, 32769])
def test_w4_activations_at_the_2gib_boundary(m):
    # M * K * 2 bytes of activations just below 2^31 (the 256 x 128
    # direct-load tile, 32-bit buffer offsets up to the last row) and just
    # above (the generic tile of the same width).
    n, g = 256, 64
    p = si.w4_problem(m, n, K, g, tag="edge-a")
    assert (p.A.nbytes < 2 ** 31) == (m == 32767)
    tiled = qg.repack_w4(to_dev(p.packed))
    C = qg.gemm_w4a16(to_dev(p.A, BF16), tiled, to_dev(p.scale, BF16), to_dev(p.zero, BF16),
                      None, g)
    torch.cuda.synchronize()
    rows, cols = _pairs(m, n, 4)
    rows = np.concatenate([rows, [m - 1, m - 2, 32766]])
    cols = np.concatenate([cols, [255, 0, 131]])
    _check(C, oracle.gemm_w4_at(p.A, p.packed, p.scale, p.zero, g, rows, cols, BF16),
           rows, cols, BF16, f"m={m}")
    del tiled, C
    torch.cuda.empty_cache()
