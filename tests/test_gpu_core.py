"""GPU parity, part 1: repack, the dequant hook, integer-exact GEMMs on every
path, and the tiny W4A16 problem against the oracle.

Every comparison runs the library through its C ABI (the binding passes raw
pointers) and compares with the CPU oracle on identical seeded bytes."""

import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
import weight_only_quantized_w8a16_amd as qg
from helpers import (BF16, FP16, TOL, rel_err, tiled_w4_expected, tiled_w8_expected, to_bits,
                     to_dev)

pytestmark = pytest.mark.gpu


# -- repack -------------------------------------------------------------------

@pytest.mark.parametrize("n,k", [(16, 128), (48, 384), (128, 256), (32, 640), (64, 896), (2048, 2048)])
def test_repack_w4_matches_documented_layout_and_inverts(n, k):
    packed = np.random.default_rng(n + k).integers(0, 256, (n, k // 2), dtype=np.uint8)
    d = to_dev(packed)
    tiled = qg.repack_w4(d)
    assert np.array_equal(tiled.cpu().numpy(), tiled_w4_expected(packed))
    back = qg.unrepack_w4(tiled)
    assert np.array_equal(back.cpu().numpy(), packed)


@pytest.mark.parametrize("bits", [4, 8])
def test_repack_by_row_chunks_equals_whole(bits):
    # The tiled layouts are tile-major over 16-row channel tiles, so repacking
    # a weight in row chunks (multiples of 16, as a loader streaming a large
    # table would) and concatenating gives the bytes of the whole repack.
    n, k = 1040, 1024
    rng = np.random.default_rng(bits)
    if bits == 4:
        src = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
        rep = qg.repack_w4
    else:
        src = rng.integers(-128, 128, (n, k)).astype(np.int8)
        rep = qg.repack_w8
    whole = rep(to_dev(src)).cpu().numpy()
    cuts = [0, 16, 400, 656, 1040]
    parts = [rep(to_dev(np.ascontiguousarray(src[a:b]))).cpu().numpy() for a, b in zip(cuts, cuts[1:])]
    assert np.array_equal(np.concatenate(parts), whole)


@pytest.mark.parametrize("n,k", [(16, 64), (32, 192), (3584, 3584)])
def test_repack_w8_matches_documented_layout_and_inverts(n, k):
    codes = np.random.default_rng(n * k).integers(-128, 128, (n, k)).astype(np.int8)
    tiled = qg.repack_w8(to_dev(codes))
    assert np.array_equal(tiled.cpu().numpy(), tiled_w8_expected(codes))
    assert np.array_equal(qg.unrepack_w8(tiled).cpu().numpy(), codes)


@pytest.mark.parametrize("n,k", [(16, 64), (48, 192), (80, 320), (208, 128), (3584, 3584)])
def test_repack_w8_kn_matches_transposed_repack_and_inverts(n, k):
    # K-major int8 [k, n] in: the same tiled bytes as repacking the [n, k]
    # transpose, from the layout formula; the inverse returns [k, n].
    codes = np.random.default_rng(n + 3 * k).integers(-128, 128, (n, k)).astype(np.int8)
    codes[0, :2] = [-128, 127]
    kn = to_dev(np.ascontiguousarray(codes.T))
    tiled = qg.repack_w8_kn(kn)
    assert tuple(tiled.shape) == (n, k)
    assert np.array_equal(tiled.cpu().numpy(), tiled_w8_expected(codes))
    assert np.array_equal(qg.unrepack_w8_kn(tiled).cpu().numpy(), codes.T)


# -- dequant hook (bit-exact) ---------------------------------------------------

@pytest.mark.parametrize("dtype", [BF16, FP16])
@pytest.mark.parametrize("group", [64, 128])
@pytest.mark.parametrize("k", [512, 640])
def test_dequant_w4_bit_exact(dtype, group, k):
    n = 96
    packed, s, z, _ = si.w4_weights(n, k, group, seed=11 + group, dtype=dtype)
    ref = oracle.dequant4(packed, s, z, group, dtype)
    tiled = qg.repack_w4(to_dev(packed))
    S, Z = to_dev(s, dtype), to_dev(z, dtype)
    W32 = qg.dequant_w4(tiled, S, Z, group, torch.float32).cpu().numpy()
    assert np.array_equal(W32.view(np.uint32), ref.view(np.uint32))
    W16 = qg.dequant_w4(tiled, S, Z, group, S.dtype)
    conv = oracle.f32_to_bf16 if dtype == BF16 else oracle.f32_to_f16
    assert np.array_equal(to_bits(W16), conv(ref))


@pytest.mark.parametrize("dtype", [FP16, BF16])
def test_dequant_w8_bit_exact(dtype):
    n, k = 64, 448
    codes, s, _ = si.w8_weights(n, k, -1, seed=5, dtype=dtype)
    codes[0, :4] = [-128, 127, 0, -1]
    ref = oracle.dequant8(codes, s, -1, dtype)
    tiled = qg.repack_w8(to_dev(codes))
    S = to_dev(s, dtype)
    W32 = qg.dequant_w8(tiled, S, torch.float32).cpu().numpy()
    assert np.array_equal(W32.view(np.uint32), ref.view(np.uint32))
    conv = oracle.f32_to_bf16 if dtype == BF16 else oracle.f32_to_f16
    assert np.array_equal(to_bits(qg.dequant_w8(tiled, S, S.dtype)), conv(ref))


@pytest.mark.parametrize("dtype", [FP16, BF16])
@pytest.mark.parametrize("group", [64, 128])
def test_dequant_w8_grouped_bit_exact(dtype, group):
    n, k = 48, 640
    codes, s, _ = si.w8_weights(n, k, group, seed=group + 1, dtype=dtype)
    codes[0, :4] = [-128, 127, 0, -1]
    ref = oracle.dequant8(codes, s, group, dtype)
    tiled = qg.repack_w8(to_dev(codes))
    S = to_dev(s, dtype)
    W32 = qg.dequant_w8(tiled, S, torch.float32, group).cpu().numpy()
    assert np.array_equal(W32.view(np.uint32), ref.view(np.uint32))
    conv = oracle.f32_to_bf16 if dtype == BF16 else oracle.f32_to_f16
    assert np.array_equal(to_bits(qg.dequant_w8(tiled, S, S.dtype, group)), conv(ref))


# -- integer-exact GEMMs: bit-exact on every path --------------------------------

def _run_w4(p, path=None):
    A = to_dev(p.A, p.dtype)
    tiled = qg.repack_w4(to_dev(p.packed))
    S = to_dev(p.scale, p.dtype)
    Z = to_dev(p.zero, p.dtype) if p.zero is not None else None
    bias = to_dev(p.bias, p.bias_dtype) if p.bias is not None else None
    if path:
        qg.set_override(path=path)
    try:
        C = qg.gemm_w4a16(A, tiled, S, Z, bias, p.group)
    finally:
        qg.set_override(path=None)
    torch.cuda.synchronize()
    return C


def _run_w8(p, path=None):
    A = to_dev(p.A, p.dtype)
    tiled = qg.repack_w8(to_dev(p.codes))
    S = to_dev(p.scale, p.dtype)
    bias = to_dev(p.bias, p.bias_dtype) if p.bias is not None else None
    if path:
        qg.set_override(path=path)
    try:
        C = qg.gemm_w8a16(A, tiled, S, bias, p.group)
    finally:
        qg.set_override(path=None)
    torch.cuda.synchronize()
    return C


def _exact_expected(Cref, dtype):
    conv = oracle.f32_to_bf16 if dtype == BF16 else oracle.f32_to_f16
    as32 = Cref.astype(np.float32)
    assert np.array_equal(as32.astype(np.float64), Cref)      # exact inputs stay exact
    return conv(as32)


@pytest.mark.parametrize("m,n,k,group", [
    (1, 16, 128, 64), (4, 128, 256, 64), (16, 48, 384, 128), (5, 2048, 2048, 64),
    (33, 128, 256, 64), (100, 192, 512, 128), (256, 256, 1024, 64), (7, 256, 640, 64),
])
@pytest.mark.parametrize("path", ["decode", "prefill"])
@pytest.mark.parametrize("dtype", [BF16, FP16])
def test_w4_integer_exact(m, n, k, group, path, dtype):
    p = si.w4_exact_problem(m, n, k, group, seed=m * 7 + n + k, dtype=dtype, bias_dtype=FP16)
    Cref = oracle.gemm_w4(p.A, p.packed, p.scale, p.zero, group, dtype, p.bias, FP16)
    C = _run_w4(p, path)
    got = to_bits(C)
    exp = _exact_expected(Cref, dtype)
    bad = np.argwhere(got != exp)
    assert bad.size == 0, f"{len(bad)} mismatches, first at {bad[:4].tolist()}"


@pytest.mark.parametrize("m,n,k", [(1, 16, 64), (3, 64, 448), (16, 3584, 3584), (40, 128, 192),
                                   (130, 256, 512),
                                   # decode with up to 16 waves over K: 28, 17 and 12 chunks
                                   (1, 3584, 3584), (4, 48, 1088), (2, 32, 1536)])
@pytest.mark.parametrize("path", ["decode", "prefill"])
@pytest.mark.parametrize("dtype", [FP16, BF16])
def test_w8_integer_exact(m, n, k, path, dtype):
    p = si.w8_exact_problem(m, n, k, seed=m + n + k, dtype=dtype, bias_dtype=FP16)
    Cref = oracle.gemm_w8(p.A, p.codes, p.scale, -1, dtype, p.bias, FP16)
    got = to_bits(_run_w8(p, path))
    exp = _exact_expected(Cref, dtype)
    bad = np.argwhere(got != exp)
    assert bad.size == 0, f"{len(bad)} mismatches, first at {bad[:4].tolist()}"


@pytest.mark.parametrize("m,n,k,group", [
    (1, 16, 128, 64), (3, 64, 448, 64), (16, 3584, 3584, 128), (40, 128, 640, 128),
    (130, 256, 512, 64), (300, 512, 640, 128),
    (1, 3584, 3584, 128), (4, 48, 1088, 64), (2, 32, 1536, 128),
])
@pytest.mark.parametrize("path", ["decode", "prefill"])
@pytest.mark.parametrize("dtype", [FP16, BF16])
def test_w8_grouped_integer_exact(m, n, k, group, path, dtype):
    # int8 codes with one scale per (channel, K-group): dyadic scales keep
    # q * s exact in 16 bits, so every path must match RNE(Cref) bitwise.
    p = si.w8_exact_problem(m, n, k, seed=m + n + k + group, dtype=dtype, bias_dtype=FP16,
                            group=group)
    Cref = oracle.gemm_w8(p.A, p.codes, p.scale, group, dtype, p.bias, FP16)
    got = to_bits(_run_w8(p, path))
    exp = _exact_expected(Cref, dtype)
    bad = np.argwhere(got != exp)
    assert bad.size == 0, f"{len(bad)} mismatches, first at {bad[:4].tolist()}"


@pytest.mark.parametrize("tile", ["D8", "D8N", "D64", "D128", "X", "L", "M", "S", "P256", "P128", "P64",
                                  "W256", "W256N", "W128", "W64", "WX", "DX"])
@pytest.mark.parametrize("group", [64, 128])
def test_prefill_tiles_w8_grouped_integer_exact(tile, group):
    p = si.w8_exact_problem(300, 512, 1024, seed=group, dtype=BF16, bias_dtype=FP16, group=group)
    Cref = oracle.gemm_w8(p.A, p.codes, p.scale, group, BF16, p.bias, FP16)
    qg.set_override(prefill_tile=tile)
    got = to_bits(_run_w8(p, "prefill"))
    assert np.array_equal(got, _exact_expected(Cref, BF16))


def test_prefill_w8_grouped_odd_group_count_falls_back():
    # K / group = 3: the direct-load tile needs pairs of groups; the generic
    # tile of the same width takes the problem.
    p = si.w8_exact_problem(300, 512, 384, seed=21, dtype=FP16, bias_dtype=FP16, group=128)
    Cref = oracle.gemm_w8(p.A, p.codes, p.scale, 128, FP16, p.bias, FP16)
    qg.set_override(prefill_tile="D8")
    got = to_bits(_run_w8(p, "prefill"))
    assert np.array_equal(got, _exact_expected(Cref, FP16))


@pytest.mark.parametrize("m", [1, 16, 1024])
@pytest.mark.parametrize("group", [64, 128])
def test_w8_grouped_random_tolerance(m, group):
    # Qwen2-7B-sized layer, random codes and scales: outputs sampled across
    # the matrix within the fp16 tolerance.
    n = k = 3584
    p = si.w8_problem(m, n, k, group=group, tag="w8g", dtype=FP16)
    C = _run_w8(p).float().cpu().numpy()
    rng = np.random.default_rng(m + group)
    rows = rng.integers(0, m, 96)
    cols = rng.integers(0, n, 96)
    ref = oracle.gemm_w8_at(p.A, p.codes, p.scale, rows, cols, group, FP16)
    err = np.abs(C[rows, cols] - ref).max() / np.abs(ref).max()
    assert err <= TOL[FP16], err


# -- int4 scale forms: per channel (group -1) and scale-only (no zeros) ----------

FORMS = [(-1, True), (-1, False), (64, False), (128, False)]


@pytest.mark.parametrize("group,zeros", FORMS)
@pytest.mark.parametrize("dtype", [BF16, FP16])
def test_dequant_w4_scale_forms_bit_exact(group, zeros, dtype):
    n, k = 48, 640
    p = si.w4_exact_problem(1, n, k, group, seed=3, dtype=dtype, zeros=zeros)
    ref = oracle.dequant4(p.packed, p.scale, p.zero, group, dtype)
    tiled = qg.repack_w4(to_dev(p.packed))
    S = to_dev(p.scale, dtype)
    Z = to_dev(p.zero, dtype) if zeros else None
    W32 = qg.dequant_w4(tiled, S, Z, group, torch.float32).cpu().numpy()
    assert np.array_equal(W32.view(np.uint32), ref.view(np.uint32))


# (1, 65536, 256) is a decode-sized problem: the decode path only.
@pytest.mark.parametrize("m,n,k,path", [
    (m, n, k, path) for (m, n, k) in [(1, 16, 128), (5, 256, 2048), (33, 128, 256), (300, 512, 640),
                                      (16, 3584, 3584), (1, 65536, 256)]
    for path in ("decode", "prefill") if not (path == "prefill" and n > 8192)])
@pytest.mark.parametrize("group,zeros", FORMS)
def test_w4_scale_forms_integer_exact(m, n, k, path, group, zeros):
    p = si.w4_exact_problem(m, n, k, group, seed=m + n + k, dtype=BF16, bias_dtype=FP16, zeros=zeros)
    Cref = oracle.gemm_w4(p.A, p.packed, p.scale, p.zero, group, BF16, p.bias, FP16)
    got = to_bits(_run_w4(p, path))
    exp = _exact_expected(Cref, BF16)
    bad = np.argwhere(got != exp)
    assert bad.size == 0, f"{len(bad)} mismatches, first at {bad[:4].tolist()}"


@pytest.mark.parametrize("tile", ["D8", "D8N", "D64", "D128", "X", "L", "M", "S", "P256", "P128", "P64"])
@pytest.mark.parametrize("group,zeros", FORMS)
def test_prefill_tiles_w4_scale_forms_exact(tile, group, zeros):
    # scale-only groups keep the direct-load tiles (their zero windows read an
    # empty buffer, i.e. zeros); per-channel scales fall back to the generic tile
    p = si.w4_exact_problem(300, 512, 1024, group, seed=29, dtype=FP16, bias_dtype=FP16, zeros=zeros)
    Cref = oracle.gemm_w4(p.A, p.packed, p.scale, p.zero, group, FP16, p.bias, FP16)
    qg.set_override(prefill_tile=tile)
    got = to_bits(_run_w4(p, "prefill"))
    assert np.array_equal(got, _exact_expected(Cref, FP16))


@pytest.mark.parametrize("group,zeros", FORMS)
def test_w4_scale_forms_random_tolerance(group, zeros):
    # random bf16 data on the decode and prefill paths, sampled outputs
    for m in (1, 256):
        p = si.w4_problem(m, 2048, 2048, group, tag="forms")
        if not zeros:
            p.zero = None
        C = _run_w4(p).float().cpu().numpy()
        rng = np.random.default_rng(m)
        rows, cols = rng.integers(0, m, 64), rng.integers(0, 2048, 64)
        ref = oracle.gemm_w4_at(p.A, p.packed, p.scale, p.zero, group, rows, cols, BF16)
        err = np.abs(C[rows, cols] - ref).max() / np.abs(ref).max()
        assert err <= TOL[BF16], (m, err)


# -- the tiny W4A16 problem (M=4, K=256, N=128, g=64), full oracle ----------------

@pytest.mark.parametrize("path", [None, "decode", "prefill"])
def test_tiny_w4a16_parity(path):
    p = si.w4_problem(4, 128, 256, 64, tag="cfg0")
    Cref = oracle.gemm_w4(p.A, p.packed, p.scale, p.zero, 64, BF16)
    C = _run_w4(p, path)
    assert C.dtype == torch.bfloat16 and tuple(C.shape) == (4, 128)
    err = rel_err(C.float().cpu().numpy(), Cref)
    assert err <= TOL[BF16], err


def test_empty_m_is_noop():
    p = si.w4_problem(1, 128, 256, 64, tag="cfg0")
    tiled = qg.repack_w4(to_dev(p.packed))
    A = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    C = qg.gemm_w4a16(A, tiled, to_dev(p.scale, BF16), to_dev(p.zero, BF16), None, 64)
    assert tuple(C.shape) == (0, 128)


# -- every prefill tile configuration, forced, on ragged M: bit-exact --------------

@pytest.mark.parametrize("tile", ["X", "L", "M", "S", "P256", "P128", "P64"])
@pytest.mark.parametrize("m", [1, 77, 300])
def test_prefill_tiles_integer_exact(tile, m):
    n, k, group = 512, 640, 128
    p = si.w4_exact_problem(m, n, k, group, seed=m + 3, dtype=BF16, bias_dtype=FP16)
    Cref = oracle.gemm_w4(p.A, p.packed, p.scale, p.zero, group, BF16, p.bias, FP16)
    qg.set_override(prefill_tile=tile)
    got = to_bits(_run_w4(p, "prefill"))
    assert np.array_equal(got, _exact_expected(Cref, BF16))


@pytest.mark.parametrize("tile", ["X", "L", "M", "S", "P256", "P128", "P64", "W256", "W256N", "W128", "W64",
                                  "WX", "DX"])
def test_prefill_tiles_w8_integer_exact(tile):
    p = si.w8_exact_problem(200, 256, 576, seed=9, dtype=FP16, bias_dtype=FP16)
    Cref = oracle.gemm_w8(p.A, p.codes, p.scale, -1, FP16, p.bias, FP16)
    qg.set_override(prefill_tile=tile)
    got = to_bits(_run_w8(p, "prefill"))
    assert np.array_equal(got, _exact_expected(Cref, FP16))


@pytest.mark.parametrize("m,n,k", [(1, 256, 128), (300, 512, 640), (513, 768, 2048), (256, 256, 384)])
@pytest.mark.parametrize("dtype", [BF16, FP16])
@pytest.mark.parametrize("tile", ["D8", "D8N", "D64", "D128", "X", "P256", "P128", "P64", "DX"])
@pytest.mark.parametrize("group", [64, 128])
def test_prefill_dma_tile_integer_exact(tile, group, m, n, k, dtype):
    p = si.w4_exact_problem(m, n, k, group, seed=m + k, dtype=dtype, bias_dtype=FP16)
    Cref = oracle.gemm_w4(p.A, p.packed, p.scale, p.zero, group, dtype, p.bias, FP16)
    qg.set_override(prefill_tile=tile)
    got = to_bits(_run_w4(p, "prefill"))
    assert np.array_equal(got, _exact_expected(Cref, dtype))


@pytest.mark.parametrize("tile", ["D8", "D8N", "D64", "D128", "X", "P256", "P128", "P64", "W256", "W256N", "W128",
                                  "W64", "WX", "DX"])
def test_prefill_dma_tile_w8_integer_exact(tile):
    p = si.w8_exact_problem(300, 512, 576, seed=4, dtype=FP16, bias_dtype=FP16)
    Cref = oracle.gemm_w8(p.A, p.codes, p.scale, -1, FP16, p.bias, FP16)
    qg.set_override(prefill_tile=tile)
    got = to_bits(_run_w8(p, "prefill"))
    assert np.array_equal(got, _exact_expected(Cref, FP16))


@pytest.mark.parametrize("tile", ["D8", "D8N"])
def test_prefill_dma_tile_odd_group_count_falls_back(tile):
    # K / group = 3: the scale windows need pairs of groups, so the generic
    # kernel of the same tile width takes the problem; results stay exact.
    p = si.w4_exact_problem(300, 512, 384, 128, seed=11, dtype=BF16, bias_dtype=FP16)
    Cref = oracle.gemm_w4(p.A, p.packed, p.scale, p.zero, 128, BF16, p.bias, FP16)
    qg.set_override(prefill_tile=tile)
    got = to_bits(_run_w4(p, "prefill"))
    assert np.array_equal(got, _exact_expected(Cref, BF16))


# -- dequantize-then-dense path ----------------------------------------------------

DENSE_TILES = ["P256", "P128", "P64"]


@pytest.mark.parametrize("tile", DENSE_TILES)
@pytest.mark.parametrize("group,zeros", [(64, True), (128, True)] + FORMS)
@pytest.mark.parametrize("dtype", [BF16, FP16])
def test_dense_path_equals_fused_tile_bitwise_w4(tile, group, zeros, dtype):
    # Random data: the dense tile accumulates the values the fused tile
    # dequantizes into LDS in the same order (unsplit, one K group), so the
    # two paths agree in every bit, ragged M included.
    p = si.w4_problem(300, 512, 1024, group, tag="dense", dtype=dtype, bias_dtype=FP16)
    if not zeros:
        p.zero = None
    qg.set_override(prefill_tile="D8")
    fused = _run_w4(p, "prefill")
    qg.set_override(prefill_tile=tile)
    dense = _run_w4(p, "prefill")
    assert torch.equal(fused.view(torch.int16), dense.view(torch.int16))


@pytest.mark.parametrize("tile", DENSE_TILES)
@pytest.mark.parametrize("group", [-1, 64, 128])
@pytest.mark.parametrize("k", [1152, 1024])
def test_dense_path_equals_fused_tile_bitwise_w8(tile, group, k):
    # k % 256 == 0: the int8 dequant stages four code blocks in LDS; else one
    # block per wave
    p = si.w8_problem(130, 768, k, group=group, tag="dense8", dtype=FP16, bias_dtype=BF16)
    qg.set_override(prefill_tile="D8")
    fused = _run_w8(p, "prefill")
    qg.set_override(prefill_tile=tile)
    dense = _run_w8(p, "prefill")
    assert torch.equal(fused.view(torch.int16), dense.view(torch.int16))


@pytest.mark.parametrize("m,n,k,group,tile", [(512, 3072, 2048, 64, "P64"), (1024, 3072, 2048, 128, "P128")])
def test_dense_path_taken_by_size_equals_forced_tile(m, n, k, group, tile):
    # 512 .. 1024 rows over a few hundred 256-wide column tiles: the automatic
    # choice is the dequantize-then-dense path (the binding allocates its
    # workspace), bit-equal to the forced dense tile; sampled outputs within
    # the bf16 tolerance of the oracle.
    p = si.w4_problem(m, n, k, group, tag="dense-auto", bias_dtype=BF16)
    auto = _run_w4(p, "prefill")
    qg.set_override(prefill_tile=tile)
    forced = _run_w4(p, "prefill")
    assert torch.equal(auto.view(torch.int16), forced.view(torch.int16))
    C = auto.float().cpu().numpy()
    rng = np.random.default_rng(m + n)
    rows, cols = rng.integers(0, m, 128), rng.integers(0, n, 128)
    ref = oracle.gemm_w4_at(p.A, p.packed, p.scale, p.zero, group, rows, cols, BF16, p.bias, BF16)
    assert np.abs(C[rows, cols] - ref).max() / np.abs(ref).max() <= TOL[BF16]


@pytest.mark.parametrize("tile", ["W256", "W256N", "W128", "W64"])
@pytest.mark.parametrize("dtype", [FP16, BF16])
@pytest.mark.parametrize("m,k", [(130, 1152), (300, 576), (1, 128)])
@pytest.mark.parametrize("group", [-1, 64, 128])
def test_w8_code_tile_equals_fused_tile_bitwise(tile, dtype, m, k, group):
    # int8 codes direct-loaded into LDS and converted after the read: the same
    # weights (exact codes, or q * s rounded once for group scales),
    # accumulated in the same order as the fused tile, with the channel scale
    # and bias applied the same way -- identical bits.
    if k % group:
        pytest.skip("k is not a multiple of the group")
    p = si.w8_problem(m, 768, k, group=group, tag="w8dir", dtype=dtype, bias_dtype=FP16)
    qg.set_override(prefill_tile="D8")
    fused = _run_w8(p, "prefill")
    qg.set_override(prefill_tile=tile)
    direct = _run_w8(p, "prefill")
    assert torch.equal(fused.view(torch.int16), direct.view(torch.int16))


@pytest.mark.parametrize("dtype", [FP16, BF16])
@pytest.mark.parametrize("m,n,k", [(520, 2048, 1152), (700, 2048, 576), (1024, 4096, 640)])
@pytest.mark.parametrize("group", [-1, 64])
def test_w8_mixed_tile_equals_fused_tile_bitwise(dtype, m, n, k, group):
    # 256 x 256 tiles for the first half of the large tiles, 128 x 128
    # quarters for the rest (those below the last row skipped), one launch:
    # the fused tile's bits (m = 520: a quarter row past the end).
    p = si.w8_problem(m, n, k, group=group, tag="w8mix", dtype=dtype, bias_dtype=FP16)
    qg.set_override(prefill_tile="D8")
    fused = _run_w8(p, "prefill")
    qg.set_override(prefill_tile="WX")
    mixed = _run_w8(p, "prefill")
    assert torch.equal(fused.view(torch.int16), mixed.view(torch.int16))


@pytest.mark.parametrize("dtype", [FP16, BF16])
@pytest.mark.parametrize("m,n,k", [(520, 2048, 1280), (1024, 4096, 512)])
@pytest.mark.parametrize("form", ["w4g64", "w4pc", "w8g128"])
def test_fused_mixed_tile_equals_fused_tile_bitwise(dtype, m, n, k, form):
    # Fused 256 x 256 tiles for the first half of the large tiles, 256 x 128
    # halves for the rest, one launch: the 256 x 256 tile's bits.  (K holds an
    # even number of groups, as the direct-load tiles need.)
    if form == "w8g128":
        p = si.w8_problem(m, n, k, group=128, tag="dmix", dtype=dtype, bias_dtype=FP16)
        run = _run_w8
    else:
        g = 64 if form == "w4g64" else -1
        p = si.w4_problem(m, n, k, g, tag="dmix", dtype=dtype, bias_dtype=FP16)
        run = _run_w4
    qg.set_override(prefill_tile="D8")
    fused = run(p, "prefill")
    qg.set_override(prefill_tile="DX")
    mixed = run(p, "prefill")
    assert torch.equal(fused.view(torch.int16), mixed.view(torch.int16))


def test_fused_mixed_tile_taken_by_size():
    # int8 group 128, m = 1024, n = 18944, k = 3584: one round of 256 x 256
    # tiles plus one of halves; no workspace; the forced form (another split
    # of the large tiles) gives the same bits; sampled outputs within the fp16
    # tolerance of the oracle.
    m, n, k = 1024, 18944, 3584
    p = si.w8_problem(m, n, k, group=128, tag="dmix-auto", dtype=FP16, bias_dtype=FP16)
    assert qg.gemm_workspace_size(m, n, k, 128, 8) == 0
    auto = _run_w8(p, "prefill")
    qg.set_override(prefill_tile="DX")
    forced = _run_w8(p, "prefill")
    assert torch.equal(auto.view(torch.int16), forced.view(torch.int16))
    C = auto.float().cpu().numpy()
    rng = np.random.default_rng(m + n)
    rows, cols = rng.integers(0, m, 96), rng.integers(0, n, 96)
    ref = oracle.gemm_w8_at(p.A, p.codes, p.scale, rows, cols, 128, FP16, p.bias, FP16)
    assert np.abs(C[rows, cols] - ref).max() / np.abs(ref).max() <= TOL[FP16]


@pytest.mark.parametrize("dtype", [FP16, BF16])
@pytest.mark.parametrize("m", [130, 64])
@pytest.mark.parametrize("group,nsplit", [(-1, 2), (-1, 3), (-1, 4), (128, 2)])
def test_w8_code_tile_k_slices_equal_fused_k_slices_bitwise(dtype, m, group, nsplit):
    # K slices on the code-converting 64 x 128 tile and on the fused 64-row
    # direct-load tile, sliced alike (K = 2048: 16 or 8 steps a slice): the
    # same fp32 partials, so the same reduced bits.
    n, k = 512, 2048
    p = si.w8_problem(m, n, k, group=group, tag="w8dir-split", dtype=dtype, bias_dtype=FP16)
    qg.set_override(prefill_tile="D64", splitk=nsplit)
    fused = _run_w8(p, "prefill")
    qg.set_override(prefill_tile="W64", splitk=nsplit)
    direct = _run_w8(p, "prefill")
    qg.set_override(splitk=None)
    assert torch.equal(fused.view(torch.int16), direct.view(torch.int16))


@pytest.mark.parametrize("m,n,tile,nsplit", [(512, 3584, "W64", 1), (1024, 3584, "W128", 1),
                                             (128, 18944, "W128", 1), (1024, 18944, "WX", 1),
                                             (128, 3584, "W64", 4), (64, 3584, "W64", 7)])
def test_w8_code_tile_taken_by_size(m, n, tile, nsplit):
    # int8 per channel, one round of 64 x 128 or 128 x 128 tiles, or whole
    # rounds of 256 x 256 tiles with at most a quarter-round left, or (up to
    # 128 rows, few 64 x 128 tiles) 64 x 128 tiles in K slices: the automatic
    # choice is the code-converting tile (workspace only for the slices'
    # partials), bit-equal to it forced (WX forced splits the large tiles
    # differently: same bits); sampled outputs within the fp16 tolerance of
    # the oracle.
    k = 3584
    p = si.w8_problem(m, n, k, group=-1, tag="w8dir-auto", dtype=FP16, bias_dtype=FP16)
    assert qg.gemm_workspace_size(m, n, k, -1, 8) == (0 if nsplit == 1 else nsplit * m * n * 4)
    auto = _run_w8(p, "prefill")
    qg.set_override(prefill_tile=tile)
    forced = _run_w8(p, "prefill")
    assert torch.equal(auto.view(torch.int16), forced.view(torch.int16))
    C = auto.float().cpu().numpy()
    rng = np.random.default_rng(m + n)
    rows, cols = rng.integers(0, m, 96), rng.integers(0, n, 96)
    ref = oracle.gemm_w8_at(p.A, p.codes, p.scale, rows, cols, -1, FP16, p.bias, FP16)
    assert np.abs(C[rows, cols] - ref).max() / np.abs(ref).max() <= TOL[FP16]


@pytest.mark.parametrize("tile", ["P256", "P128", "P64", "W256", "W128", "W64"])
def test_forced_wide_tile_ignored_when_n_does_not_fit(tile):
    # n = 272 (17 channel tiles of 16) fits none of these tiles' widths: the
    # forced choice is ignored and the call runs as if nothing were forced.
    p8 = si.w8_problem(300, 272, 576, group=-1, tag="w8-odd-n", dtype=FP16, bias_dtype=FP16)
    p4 = si.w4_problem(300, 272, 640, 64, tag="w4-odd-n", bias_dtype=BF16)
    auto8, auto4 = _run_w8(p8, "prefill"), _run_w4(p4, "prefill")
    qg.set_override(prefill_tile=tile)
    assert qg.gemm_workspace_size(300, 272, 640, 64, 4) == 0
    forced8, forced4 = _run_w8(p8, "prefill"), _run_w4(p4, "prefill")
    assert torch.equal(auto8.view(torch.int16), forced8.view(torch.int16))
    assert torch.equal(auto4.view(torch.int16), forced4.view(torch.int16))


@pytest.mark.parametrize("tile", DENSE_TILES)
def test_dense_path_workspace_size_and_fallback(tile):
    # The dense path asks for n * k 16-bit values of workspace; with less the
    # call runs the fused tiles, bit-equal to the automatic choice.
    m, n, k, group = 200, 256, 640, 64
    p = si.w4_problem(m, n, k, group, tag="dense-ws")
    A = to_dev(p.A, p.dtype)
    tiled = qg.repack_w4(to_dev(p.packed))
    S, Z = to_dev(p.scale, p.dtype), to_dev(p.zero, p.dtype)
    qg.set_override(path="prefill")
    auto = qg.gemm_w4a16(A, tiled, S, Z, None, group)
    qg.set_override(prefill_tile=tile)
    need = int(qg.lib().qgemm_workspace_size(m, n, k, group, 4))
    assert need == n * k * 2
    small = torch.empty(need - 256, dtype=torch.uint8, device="cuda")
    fallback = qg.gemm_w4a16(A, tiled, S, Z, None, group, workspace=small)
    full = torch.empty(need, dtype=torch.uint8, device="cuda")
    dense = qg.gemm_w4a16(A, tiled, S, Z, None, group, workspace=full)
    torch.cuda.synchronize()
    assert torch.equal(auto.view(torch.int16), fallback.view(torch.int16))
    ref = oracle.gemm_w4(p.A, p.packed, p.scale, p.zero, group, BF16)
    assert rel_err(dense.float().cpu().numpy(), ref) <= TOL[BF16]


@pytest.mark.parametrize("nbytes", [0, 16, 4096 + 48, 10 * (1 << 20) + 160])
def test_read_probe_reads_every_byte_once(nbytes):
    # The streaming-read probe XOR-folds what it reads; the XOR of its
    # per-workgroup words equals the XOR of every 32-bit word of the range.
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 2 ** 32, (nbytes + 64) // 4, dtype=np.uint32)
    buf = to_dev(host)
    blocks = int(qg.lib().qg_read_probe_blocks(nbytes))
    out = torch.zeros(blocks, dtype=torch.int32, device="cuda")
    qg.read_probe(buf if nbytes else None, nbytes, out)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(host[: nbytes // 4]) if nbytes else np.uint32(0)
    assert got == want


@pytest.mark.parametrize("waves", [4, 8, 16])
def test_lds_probe_counts_cycles(waves):
    # One workgroup per CU reading its LDS: every workgroup reports a loop of
    # at least one clock per 256 bytes (the widest an LDS could serve) and
    # well under a second's worth of cycles.
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    iters = 1024
    cyc = torch.zeros(cus, dtype=torch.int64, device="cuda")
    qg.lds_probe(waves, iters, cyc)
    torch.cuda.synchronize()
    c = cyc.cpu().numpy()
    floor = iters * waves * 1024 / 256
    assert (c >= floor).all() and (c < 2e9).all(), (c.min(), c.max(), floor)


@pytest.mark.parametrize("m", [1, 2, 3, 4, 7, 8])
@pytest.mark.parametrize("group,dtype", [(64, BF16), (128, FP16)])
def test_large_n_decode_integer_exact(m, group, dtype):
    # Many channel tiles (N = 65536): one or two rows run the streaming decode
    # kernel, more rows the split-K one; on integer-exact inputs every output
    # is RNE of the exact sum.
    n, k = 65536, 2048
    p = si.w4_exact_problem(m, n, k, group, seed=m * 7 + group, dtype=dtype, bias_dtype=FP16)
    C = to_bits(_run_w4(p))
    rows = np.arange(m)
    cols = np.unique(np.concatenate([[0, 15, 16, n - 1], np.random.default_rng(m).integers(0, n, 300)]))
    r, c = np.meshgrid(rows, cols, indexing="ij")
    ref = oracle.gemm_w4_at(p.A, p.packed, p.scale, p.zero, group, r.ravel(), c.ravel(), dtype,
                            p.bias, FP16)
    assert np.array_equal(C[r.ravel(), c.ravel()], _exact_expected(ref, dtype))
