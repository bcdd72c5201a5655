"""GPU parity: the groupwise min/max int4 quantizer against the CPU oracle.

Codes, scales and zeros are decided in fp32 on both sides (correctly rounded
division, ties to even), so they must agree bit for bit; 16-bit scales and
zeros are the oracle's fp32 values rounded to nearest even."""
import numpy as np
import pytest
import torch

import oracle
import weight_only_quantized_w8a16_amd as qg

pytestmark = pytest.mark.gpu

DT = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}


def weights(n, k, group, dtype, seed):
    """Gaussian rows of varied spread, plus rows that exercise the edge
    cases: a constant row, dyadic grid values with exact ties, and a row with
    one outlier per group."""
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((n, k)) * rng.uniform(0.005, 3.0, (n, 1))
    if n >= 4:
        w[0] = -0.375
        grid = rng.integers(0, 31, k) / 2.0          # halves: ties at every odd value
        grid[::group] = 0.0
        grid[1::group] = 15.0
        w[1] = grid - 4.0
        w[2] = rng.standard_normal(k) * 0.01
        w[2, 5::group] = 40.0
    t = torch.from_numpy(w.astype(np.float32)).to(DT[dtype])
    return t, t.float().numpy()


def expected_sz(v, sz):
    if sz == "fp32":
        return v.view(np.uint32)
    return oracle.f32_to_bf16(v) if sz == "bf16" else oracle.f32_to_f16(v)


def got_bits(t):
    a = t.cpu()
    if a.dtype == torch.float32:
        return a.numpy().view(np.uint32)
    return a.view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("n,k", [(4, 128), (7, 640), (48, 1024), (300, 2048)])
@pytest.mark.parametrize("group", [64, 128])
@pytest.mark.parametrize("wdt", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("sz", ["fp32", "bf16", "fp16"])
def test_quantize_w4_bit_exact(n, k, group, wdt, sz):
    W, w32 = weights(n, k, group, wdt, seed=n + k + group)
    packed, s, z = qg.quantize_w4(W.cuda(), group, DT[sz])
    torch.cuda.synchronize()
    rp, rs, rz = oracle.quantize4(w32, group)
    assert np.array_equal(packed.cpu().numpy(), rp)
    assert np.array_equal(got_bits(s), expected_sz(rs, sz))
    assert np.array_equal(got_bits(z), expected_sz(rz, sz))


def test_quantize_w4_grid_and_ties_closed_form():
    # Values lo + q * step (each group holding q = 0 and 15) come back as q;
    # a group with lo = 0, hi = 15 sends halves to the even code.
    rng = np.random.default_rng(3)
    n, k, g = 32, 512, 64
    q = rng.integers(0, 16, (n, k))
    q[:, ::g] = 0
    q[:, 1::g] = 15
    step = 2.0 ** -rng.integers(2, 7, (n, k // g))
    lo = rng.integers(-32, 33, (n, k // g)) / 8.0
    w = np.repeat(lo, g, axis=1) + q * np.repeat(step, g, axis=1)
    w[0, :64] = 0.0
    w[0, 1] = 15.0
    w[0, 2:7] = [0.5, 1.5, 2.5, 13.5, 14.5]
    q[0, :64] = 0
    q[0, 1] = 15
    q[0, 2:7] = [0, 2, 2, 14, 14]
    packed, s, z = qg.quantize_w4(torch.from_numpy(w.astype(np.float32)).cuda(), g, torch.float32)
    assert np.array_equal(oracle.unpack4(packed.cpu().numpy()), q)


def test_quantize_w4_full_size_sampled_rows():
    # The tied-vocabulary projection, 131072 x 2048 bf16, quantized as one
    # launch; rows are independent, so sampled rows are checked exactly.
    n, k, g = 131072, 2048, 64
    gen = torch.Generator(device="cuda")
    gen.manual_seed(17)
    W = (torch.randn(n, k, device="cuda", generator=gen) * 0.02).to(torch.bfloat16)
    packed, s, z = qg.quantize_w4(W, g)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(16), np.arange(n - 16, n),
                                     np.random.default_rng(5).integers(0, n, 200)]))
    idx = torch.from_numpy(rows).cuda()
    rp, rs, rz = oracle.quantize4(W[idx].float().cpu().numpy(), g)
    assert np.array_equal(packed[idx].cpu().numpy(), rp)
    assert np.array_equal(got_bits(s[idx]), oracle.f32_to_bf16(rs))
    assert np.array_equal(got_bits(z[idx]), oracle.f32_to_bf16(rz))


def test_quantize_repack_gemm_chain():
    # quantize -> repack -> GEMM against the oracle GEMM on the same codes.
    m, n, k, g = 5, 256, 1024, 128
    rng = np.random.default_rng(8)
    W = torch.from_numpy((rng.standard_normal((n, k)) * 0.05).astype(np.float32)).to(torch.bfloat16)
    A = torch.from_numpy(rng.standard_normal((m, k)).astype(np.float32)).to(torch.bfloat16)
    packed, s, z = qg.quantize_w4(W.cuda(), g)
    C = qg.gemm_w4a16(A.cuda(), qg.repack_w4(packed), s, z, None, g)
    torch.cuda.synchronize()
    ref = oracle.gemm_w4(A.view(torch.int16).numpy().view(np.uint16), packed.cpu().numpy(),
                         got_bits(s), got_bits(z), g, oracle.BF16)
    err = np.abs(C.float().cpu().numpy() - ref).max() / np.abs(ref).max()
    assert err <= 1e-2, err
