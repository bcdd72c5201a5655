"""GPU parity of the split-K prefill path: K slices write fp32 partials to
the caller's workspace and one reduction sums them in slice order.  On
integer-exact inputs every summation order gives the same fp32 value, so
every tile, slice count and weight format must match the oracle bitwise."""
import os

import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
import weight_only_quantized_w8a16_amd as qg
from helpers import BF16, FP16, to_bits, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _prefill_only():
    qg.set_override(path="prefill")


def expected(Cref, dtype):
    conv = oracle.f32_to_bf16 if dtype == BF16 else oracle.f32_to_f16
    return conv(Cref.astype(np.float32))


def _bias(p):
    return to_dev(p.bias, p.bias_dtype) if p.bias is not None else None


def run_w4(p, workspace=None):
    C = qg.gemm_w4a16(to_dev(p.A, p.dtype), qg.repack_w4(to_dev(p.packed)), to_dev(p.scale, p.dtype),
                      to_dev(p.zero, p.dtype), _bias(p), p.group, workspace=workspace)
    torch.cuda.synchronize()
    return to_bits(C)


def run_w8(p, workspace=None):
    C = qg.gemm_w8a16(to_dev(p.A, p.dtype), qg.repack_w8(to_dev(p.codes)), to_dev(p.scale, p.dtype),
                      _bias(p), p.group, workspace=workspace)
    torch.cuda.synchronize()
    return to_bits(C)


@pytest.mark.parametrize("tile", ["D8", "D8N", "D64", "D128", "X", "L", "M", "S"])
@pytest.mark.parametrize("slices", [2, 3, 4])
@pytest.mark.parametrize("group", [64, 128, -1])
def test_split_w4_every_tile_exact(tile, slices, group):
    # K = 4096: 64 steps, so with 128-groups (16-step windows) 3 and 4
    # slices still give more than one slice; M and N ragged against tiles.
    p = si.w4_exact_problem(300, 768, 4096, group, seed=slices + group, dtype=BF16, bias_dtype=FP16)
    Cref = oracle.gemm_w4(p.A, p.packed, p.scale, p.zero, group, BF16, p.bias, FP16)
    qg.set_override(prefill_tile=tile)
    qg.set_override(splitk=slices)
    assert np.array_equal(run_w4(p), expected(Cref, BF16))


@pytest.mark.parametrize("tile", ["D8", "D8N", "D64", "D128", "X", "L", "M", "S"])
@pytest.mark.parametrize("group", [-1, 128])
def test_split_w8_every_tile_exact(tile, group):
    p = si.w8_exact_problem(200, 512, 3584, seed=7, dtype=FP16, bias_dtype=FP16, group=group)
    Cref = oracle.gemm_w8(p.A, p.codes, p.scale, group, FP16, p.bias, FP16)
    qg.set_override(prefill_tile=tile)
    qg.set_override(splitk=3)
    assert np.array_equal(run_w8(p), expected(Cref, FP16))


def test_automatic_split_shape_and_small_workspace():
    # M = 128, N = 3072, K = 2048: the plan splits K in two (the library asks
    # for workspace); with too little workspace the call runs unsplit.  Both
    # give the exact result.
    m, n, k, g = 128, 3072, 2048, 64
    assert qg.gemm_workspace_size(m, n, k, g, 4) == 2 * m * n * 4
    p = si.w4_exact_problem(m, n, k, g, seed=5, dtype=BF16, bias_dtype=FP16)
    exp = expected(oracle.gemm_w4(p.A, p.packed, p.scale, p.zero, g, BF16, p.bias, FP16), BF16)
    assert np.array_equal(run_w4(p), exp)
    small = torch.empty(1024, dtype=torch.uint8, device="cuda")
    assert np.array_equal(run_w4(p, workspace=small), exp)


def test_split_random_data_within_tolerance():
    # Random bf16 data: the split result stays within the bf16 tolerance of
    # the oracle (only the fp32 summation order differs from unsplit).
    p = si.w4_problem(96, 1024, 4096, 64, tag="split")
    Cref = oracle.gemm_w4(p.A, p.packed, p.scale, p.zero, 64, BF16)
    qg.set_override(splitk=4)
    got = run_w4(p)
    C = torch.from_numpy(got.view(np.int16)).view(torch.bfloat16).float().numpy()
    err = np.abs(C - Cref).max() / np.abs(Cref).max()
    assert err <= 1e-2, err


@pytest.mark.parametrize("n,split", [(4032, True), (8128, True), (8192, False), (13312, False)])
def test_split_threshold_by_tile_count(n, split):
    # M = 128 on the 64 x 64 tile splits K only while those tiles number
    # fewer than 256 (2 x 127 = 254 splits, 2 x 128 = 256 does not); both
    # sides give the exact result.
    m, k, g = 128, 2048, 64
    ws = qg.gemm_workspace_size(m, n, k, g, 4)
    assert (ws > 0) == split, (n, ws)
    p = si.w4_exact_problem(m, n, k, g, seed=n, dtype=BF16, bias_dtype=FP16)
    exp = expected(oracle.gemm_w4(p.A, p.packed, p.scale, p.zero, g, BF16, p.bias, FP16), BF16)
    assert np.array_equal(run_w4(p), exp)


# -- the 64 x 64 tile's two K groups on uneven step counts ------------------------

@pytest.mark.parametrize("k,slices", [(64, 1), (192, 1), (576, 1), (576, 2), (576, 3), (1088, 2)])
def test_k_groups_uneven_steps_w8_exact(k, slices):
    # The 64 x 64 tile splits each slice's 64-k steps between two K groups of
    # waves: K = 64 leaves the second group no step, 192 and 576 (3 and 9
    # steps) give it one fewer than the first; with 8-step slices 576 splits
    # 8 + 1 and 1088 (17 steps) 16 + 1, so a one-step slice again leaves the
    # second group idle.  Integer-exact inputs: bitwise equal to the oracle.
    p = si.w8_exact_problem(40, 192, k, seed=k + slices, dtype=FP16, bias_dtype=FP16)
    Cref = oracle.gemm_w8(p.A, p.codes, p.scale, -1, FP16, p.bias, FP16)
    qg.set_override(prefill_tile="S")
    qg.set_override(splitk=slices)
    assert np.array_equal(run_w8(p), expected(Cref, FP16))


@pytest.mark.parametrize("k", [128, 384])
def test_k_groups_w4_short_k_exact(k):
    # W4 with 2 and 6 steps: one and three steps per K group.
    p = si.w4_exact_problem(70, 128, k, 64, seed=k, dtype=BF16, bias_dtype=FP16)
    Cref = oracle.gemm_w4(p.A, p.packed, p.scale, p.zero, 64, BF16, p.bias, FP16)
    qg.set_override(prefill_tile="S")
    assert np.array_equal(run_w4(p), expected(Cref, BF16))
