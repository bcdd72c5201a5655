"""GPU parity, part 2: every workload configuration against the CPU oracle.

Small problems are compared in full.  At full size the oracle evaluates a
sample of outputs one by one (first/last rows and columns, tile edges, and
random positions) in the launch configuration the benchmark uses."""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
import weight_only_quantized_w8a16_amd as qg
from helpers import BF16, FP16, TOL, TORCH_DT, rel_err, to_bits, to_dev

pytestmark = pytest.mark.gpu


def sample_pairs(m, n, seed, grid_rows=6, grid_cols=192, rand=512):
    rng = np.random.default_rng(seed)
    rows = np.unique(np.concatenate([[0, m - 1, m // 2], rng.integers(0, m, grid_rows)]))
    cols = np.unique(np.concatenate([[0, n - 1, n - 16, 63, 64, 127, 128],
                                     rng.integers(0, n, grid_cols)]))
    cols = cols[(cols >= 0) & (cols < n)]
    rr, cc = np.meshgrid(rows, cols, indexing="ij")
    r = np.concatenate([rr.ravel(), rng.integers(0, m, rand)])
    c = np.concatenate([cc.ravel(), rng.integers(0, n, rand)])
    return r, c


def _nan_out(m, n, dtype):
    """An output buffer filled with NaN: a finite result everywhere proves
    the kernels wrote every element (the sampled checks below cannot)."""
    return torch.full((m, n), float("nan"), dtype=TORCH_DT[dtype], device="cuda")


def gpu_w4(p):
    A = to_dev(p.A, p.dtype)
    tiled = qg.repack_w4(to_dev(p.packed))
    bias = to_dev(p.bias, p.bias_dtype) if p.bias is not None else None
    Z = to_dev(p.zero, p.dtype) if p.zero is not None else None
    C = qg.gemm_w4a16(A, tiled, to_dev(p.scale, p.dtype), Z, bias, p.group,
                      out=_nan_out(p.m, p.n, p.dtype))
    assert bool(torch.isfinite(C).all()), "an output element was never written"
    return C.float().cpu().numpy()


def gpu_w8(p):
    A = to_dev(p.A, p.dtype)
    tiled = qg.repack_w8(to_dev(p.codes))
    bias = to_dev(p.bias, p.bias_dtype) if p.bias is not None else None
    C = qg.gemm_w8a16(A, tiled, to_dev(p.scale, p.dtype), bias, p.group,
                      out=_nan_out(p.m, p.n, p.dtype))
    assert bool(torch.isfinite(C).all()), "an output element was never written"
    return C.float().cpu().numpy()


# -- W4A16 decode sweep: K=2048, g=64, M in {1,2,4,8}, N in {2048,3072,13312},
#    plus the tied-vocab projection N=131072 at M=1.  Full oracle.
@pytest.mark.parametrize("m,n", [(m, n) for m in (1, 2, 4, 8) for n in (2048, 3072, 13312)]
                         + [(1, 131072)])
def test_decode_sweep(m, n):
    p = si.w4_problem(m, n, 2048, 64, tag="cfg1")
    Cref = oracle.gemm_w4(p.A, p.packed, p.scale, p.zero, 64)
    err = rel_err(gpu_w4(p), Cref)
    assert err <= TOL[BF16], (m, n, err)


# -- W8A16 per channel: fp16, K=3584, N in {3584, 18944}, M in {1,16,128,1024,4096}
@pytest.mark.parametrize("m", [1, 16, 128, 1024, 4096])
@pytest.mark.parametrize("n", [3584, 18944])
def test_w8a16_per_channel(m, n):
    p = si.w8_problem(m, n, 3584, -1, tag="cfg2")
    C = gpu_w8(p)
    if m * n <= 16 * 18944 or (m, n) == (128, 3584):
        Cref = oracle.gemm_w8(p.A, p.codes, p.scale, -1, FP16)
        err = rel_err(C, Cref)
    else:
        r, c = sample_pairs(m, n, seed=m + n)
        ref = oracle.gemm_w8_at(p.A, p.codes, p.scale, r, c, -1, FP16)
        err = rel_err(C[r, c], ref)
    assert err <= TOL[FP16], (m, n, err)
    assert np.isfinite(C).all()


# -- W4A16 prefill: M in {512, 2048}, K=2048, N in {3072, 13312, 131072},
#    g in {64, 128}, fp16 bias, bf16 output.
@pytest.mark.parametrize("g", [64, 128])
@pytest.mark.parametrize("m,n", [(512, 3072), (512, 13312), (512, 131072), (2048, 3072),
                                 (2048, 13312), (2048, 131072)])
def test_prefill(m, n, g):
    p = si.w4_problem(m, n, 2048, g, tag="cfg3", bias_dtype=FP16, scale_range=(0.005, 0.02))
    C = gpu_w4(p)
    if (m, n) == (512, 3072):
        Cref = oracle.gemm_w4(p.A, p.packed, p.scale, p.zero, g, BF16, p.bias, FP16)
        err = rel_err(C, Cref)
    else:
        r, c = sample_pairs(m, n, seed=m * 3 + n + g)
        ref = oracle.gemm_w4_at(p.A, p.packed, p.scale, p.zero, g, r, c, BF16, p.bias, FP16)
        err = rel_err(C[r, c], ref)
    assert err <= TOL[BF16], (m, n, g, err)


def test_prefill_integer_exact_at_the_metric_shape():
    # M = 512, N = 131072, K = 2048, g = 64 with an fp16 bias, on the tile
    # and grouped per-XCD tile order the benchmark times: dyadic inputs make
    # every partial sum exact in fp32, so all 67M outputs must equal the
    # round-to-nearest-even of the exact product bit for bit.  The exact
    # product is the oracle's dequantized weight times A in fp64 (exact for
    # these inputs), a library matmul as the brute-force step.
    m, n, k, g = 512, 131072, 2048, 64
    p = si.w4_exact_problem(m, n, k, g, seed=512, dtype=BF16, bias_dtype=FP16)
    A = to_dev(p.A, BF16)
    tiled = qg.repack_w4(to_dev(p.packed))
    C = qg.gemm_w4a16(A, tiled, to_dev(p.scale, BF16), to_dev(p.zero, BF16),
                      to_dev(p.bias, FP16), g, out=_nan_out(m, n, BF16))
    got = to_bits(C)
    W = oracle.dequant4(p.packed, p.scale, p.zero, g, BF16).astype(np.float64)
    Cref = oracle.bf16_to_f32(p.A).astype(np.float64) @ W.T + oracle.f16_to_f32(p.bias)
    del W
    assert np.array_equal(Cref.astype(np.float32).astype(np.float64), Cref)
    r, c = sample_pairs(m, n, seed=5)
    at = oracle.gemm_w4_at(p.A, p.packed, p.scale, p.zero, g, r, c, BF16, p.bias, FP16)
    assert np.array_equal(at, Cref[r, c])           # the sum agrees with the oracle's own
    exp = torch.from_numpy(Cref.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
    assert np.array_equal(got.view(np.int16), exp)


# -- ragged and edge shapes ------------------------------------------------------------
@pytest.mark.parametrize("m", [1, 7, 16, 17, 31, 65, 129, 200, 257, 513])
def test_ragged_m_w4(m):
    p = si.w4_problem(m, 384, 640, 128, tag="ragged", bias_dtype=BF16)
    Cref = oracle.gemm_w4(p.A, p.packed, p.scale, p.zero, 128, BF16, p.bias, BF16)
    assert rel_err(gpu_w4(p), Cref) <= TOL[BF16]


@pytest.mark.parametrize("n", [16, 48, 80, 208])
def test_n_not_multiple_of_64_uses_row_slabs(n):
    p = si.w4_problem(40, n, 256, 64, tag="narrow")
    Cref = oracle.gemm_w4(p.A, p.packed, p.scale, p.zero, 64)
    assert rel_err(gpu_w4(p), Cref) <= TOL[BF16]


@pytest.mark.parametrize("m", [1, 5, 64])
def test_fp16_w4_and_bf16_w8(m):
    p4 = si.w4_problem(m, 256, 512, 64, tag="mix", dtype=FP16, bias_dtype=FP16)
    Cref = oracle.gemm_w4(p4.A, p4.packed, p4.scale, p4.zero, 64, FP16, p4.bias, FP16)
    assert rel_err(gpu_w4(p4), Cref) <= TOL[FP16]
    p8 = si.w8_problem(m, 256, 512, -1, tag="mix", dtype=BF16, bias_dtype=BF16)
    Cref = oracle.gemm_w8(p8.A, p8.codes, p8.scale, -1, BF16, p8.bias, BF16)
    assert rel_err(gpu_w8(p8), Cref) <= TOL[BF16]


def test_leading_dims_are_flattened():
    p = si.w4_problem(6, 128, 256, 64, tag="lead")
    A = to_dev(p.A, BF16).reshape(2, 3, 256)
    tiled = qg.repack_w4(to_dev(p.packed))
    C = qg.gemm_w4a16(A, tiled, to_dev(p.scale, BF16), to_dev(p.zero, BF16), None, 64)
    assert tuple(C.shape) == (2, 3, 128)
    Cref = oracle.gemm_w4(p.A, p.packed, p.scale, p.zero, 64)
    assert rel_err(C.reshape(6, 128).float().cpu().numpy(), Cref) <= TOL[BF16]


def test_repeated_calls_are_deterministic():
    p = si.w4_problem(8, 2048, 2048, 64, tag="det")
    a = gpu_w4(p)
    b = gpu_w4(p)
    assert np.array_equal(a, b)


# -- the streaming decode kernel (M <= 2 with many channel tiles) and its
#    fallbacks: unaligned scale rows, K not a multiple of 512, bias.
@pytest.mark.parametrize("m,n,k,g,bias", [
    (1, 65536, 2048, 64, False), (2, 65536, 2048, 128, True), (1, 65536, 512, 64, True),
    (2, 65536, 4096, 64, False), (1, 65536, 1152, 128, False), (3, 65536, 2048, 64, True),
    (4, 65536, 2048, 64, False), (5, 65536, 2048, 128, True), (8, 65536, 2048, 64, True),
    (8, 65536, 4096, 64, False), (6, 131072, 2048, 64, False),
])
def test_large_n_decode(m, n, k, g, bias):
    p = si.w4_problem(m, n, k, g, tag="stream", bias_dtype=FP16 if bias else si.NONE)
    C = gpu_w4(p)
    r, c = sample_pairs(m, n, seed=n + k + g)
    ref = oracle.gemm_w4_at(p.A, p.packed, p.scale, p.zero, g, r, c, BF16, p.bias,
                            FP16 if bias else si.NONE)
    assert rel_err(C[r, c], ref) <= TOL[BF16]


def test_unaligned_scale_rows_fall_back():
    p = si.w4_problem(1, 65536, 2048, 64, tag="unal")
    A = to_dev(p.A, BF16)
    tiled = qg.repack_w4(to_dev(p.packed))

    def shifted(bits):
        buf = torch.empty(bits.size + 1, dtype=torch.bfloat16, device="cuda")
        view = buf[1:].view(bits.shape)              # 2-byte aligned, not 16
        view.copy_(to_dev(bits, BF16))
        return view
    S, Z = shifted(p.scale), shifted(p.zero)
    assert S.data_ptr() % 16 != 0
    C = qg.gemm_w4a16(A, tiled, S, Z, None, 64).float().cpu().numpy()
    r, c = sample_pairs(1, 65536, seed=3)
    ref = oracle.gemm_w4_at(p.A, p.packed, p.scale, p.zero, 64, r, c)
    assert rel_err(C[r, c], ref) <= TOL[BF16]


# -- The direct-load prefill tiles bring the tile's bias and int8 channel
#    scales into LDS with 4-byte direct loads; a pointer that is only 2-byte
#    aligned keeps the per-element global loads.  Both paths give the same bits,
#    and both match the oracle.  M = 512, N = 4096 runs the 256 x 256 tile.
def _shifted(t):
    buf = torch.empty(t.numel() + 1, dtype=t.dtype, device="cuda")
    view = buf[1:].view(t.shape)                     # 2-byte aligned
    view.copy_(t)
    assert view.data_ptr() % 4 != 0
    return view


@pytest.mark.parametrize("bits", [4, 8])
def test_prefill_epilogue_constants_unaligned(bits):
    m, n, k = 512, 4096, 512
    r, c = sample_pairs(m, n, seed=bits + 11)
    if bits == 4:
        p = si.w4_problem(m, n, k, 64, tag="epi-unal", bias_dtype=FP16)
        A, tiled = to_dev(p.A, BF16), qg.repack_w4(to_dev(p.packed))
        S, Z, b = to_dev(p.scale, BF16), to_dev(p.zero, BF16), to_dev(p.bias, FP16)
        C0 = qg.gemm_w4a16(A, tiled, S, Z, b, 64)
        C1 = qg.gemm_w4a16(A, tiled, S, Z, _shifted(b), 64)
        ref = oracle.gemm_w4_at(p.A, p.packed, p.scale, p.zero, 64, r, c, BF16, p.bias, FP16)
        tol = TOL[BF16]
    else:
        p = si.w8_problem(m, n, k, tag="epi-unal", bias_dtype=FP16)
        A, tiled = to_dev(p.A, FP16), qg.repack_w8(to_dev(p.codes))
        S, b = to_dev(p.scale, FP16), to_dev(p.bias, FP16)
        C0 = qg.gemm_w8a16(A, tiled, S, b, -1)
        C1 = qg.gemm_w8a16(A, tiled, _shifted(S), _shifted(b), -1)
        ref = oracle.gemm_w8_at(p.A, p.codes, p.scale, r, c, -1, FP16, p.bias, FP16)
        tol = TOL[FP16]
    assert np.array_equal(to_bits(C0), to_bits(C1))
    assert rel_err(C0.float().cpu().numpy()[r, c], ref) <= tol


# -- Tile-choice boundaries: M just below / above each rule of the prefill
#    dispatch, at a width where the direct-load tiles are eligible.  Sampled
#    outputs against the oracle (K small to keep the oracle quick).
@pytest.mark.parametrize("m", [17, 64, 65, 128, 129, 192, 193, 256, 257])
@pytest.mark.parametrize("bits", [4, 8])
def test_prefill_dispatch_boundaries(m, bits):
    n, k = 65536, 256
    r, c = sample_pairs(m, n, seed=m + bits, grid_rows=4, grid_cols=64, rand=256)
    if bits == 4:
        p = si.w4_problem(m, n, k, 64, tag="dispatch", bias_dtype=FP16)
        got = gpu_w4(p)[r, c]
        ref = oracle.gemm_w4_at(p.A, p.packed, p.scale, p.zero, 64, r, c, BF16, p.bias, FP16)
        tol = TOL[BF16]
    else:
        p = si.w8_problem(m, n, k, tag="dispatch", bias_dtype=FP16)
        got = gpu_w8(p)[r, c]
        ref = oracle.gemm_w8_at(p.A, p.codes, p.scale, r, c, -1, FP16, p.bias, FP16)
        tol = TOL[FP16]
    err = np.abs(got - ref).max() / np.abs(ref).max()
    assert err <= tol, (m, bits, err)
