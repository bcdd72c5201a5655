"""GPU parity of the quantized embedding lookup (vllm-omni cpu_int4.py,
CPUInt4EmbeddingMethod.embedding) against the oracle: bit-exact, since the
lookup is the dequant rule (one fp32 rounding) followed by one rounding to the
output dtype.  The tiled table is the same tensor the lm_head GEMM reads."""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
import weight_only_quantized_w8a16_amd as qg
from helpers import BF16, FP16, TORCH_DT, to_bits, to_dev

pytestmark = pytest.mark.gpu


def ids_for(vocab, tokens, seed):
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, vocab, tokens).astype(np.int32)
    ids[: min(tokens, 4)] = [vocab - 1, 0, vocab - 1, 0][: min(tokens, 4)]    # repeats, both ends
    if tokens >= 8:
        ids[4:8] = [-1, vocab, 2 ** 31 - 1, -(2 ** 31)]                      # outside the table
    return ids


def expect16(vals, dt):
    return oracle.f32_to_bf16(vals) if dt == BF16 else oracle.f32_to_f16(vals)


@pytest.mark.parametrize("tiled", [True, False])
@pytest.mark.parametrize("dt", [BF16, FP16])
@pytest.mark.parametrize("group,zeros", [(64, True), (128, True), (64, False), (-1, True), (-1, False)])
@pytest.mark.parametrize("vocab,hidden,tokens", [(48, 256, 9), (160, 640, 37)])
def test_embed_w4_bit_exact(tiled, dt, group, zeros, vocab, hidden, tokens):
    packed, s, z, _ = si.w4_weights(vocab, hidden, group, si.seed_of("emb4", vocab, hidden, group), dt)
    ids = ids_for(vocab, tokens, vocab + hidden)
    table = to_dev(packed)
    if tiled:
        table = qg.repack_w4(table)
    S, Z = to_dev(s, dt), (to_dev(z, dt) if zeros else None)
    g = hidden if group == -1 else group
    ref = oracle.embed4(ids, packed, s, z if zeros else None, g, dt)
    d_ids = to_dev(ids)
    out16 = qg.embed_w4(d_ids, table, S, Z, group, tiled=tiled)
    out32 = qg.embed_w4(d_ids, table, S, Z, group, tiled=tiled, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert out16.dtype == TORCH_DT[dt] and out16.shape == (tokens, hidden)
    assert np.array_equal(out32.cpu().numpy(), ref)
    assert np.array_equal(to_bits(out16), expect16(ref, dt))


@pytest.mark.parametrize("tiled", [True, False])
@pytest.mark.parametrize("group", [-1, 64, 128])
def test_embed_w8_bit_exact(tiled, group):
    vocab, hidden, tokens = 64, 384, 21
    codes, s, _ = si.w8_weights(vocab, hidden, group, si.seed_of("emb8", vocab, hidden, group))
    codes[0, :2] = [-128, 127]
    ids = ids_for(vocab, tokens, group + 7)
    table = to_dev(codes)
    if tiled:
        table = qg.repack_w8(table)
    ref = oracle.embed8(ids, codes, s, group, FP16)
    d_ids = to_dev(ids)
    out16 = qg.embed_w8(d_ids, table, to_dev(s, FP16), group, tiled=tiled)
    out32 = qg.embed_w8(d_ids, table, to_dev(s, FP16), group, tiled=tiled, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert np.array_equal(out32.cpu().numpy(), ref)
    assert np.array_equal(to_bits(out16), expect16(ref, FP16))


def test_tied_table_serves_lookup_and_lm_head():
    # One tiled int4 copy: the lookup returns the rows the dequant hook gives,
    # and the same tensor is the lm_head GEMM weight (checked elsewhere).
    vocab, hidden = 4096, 2048
    packed, s, z, _ = si.w4_weights(vocab, hidden, 64, si.seed_of("tied", vocab, hidden))
    tiled = qg.repack_w4(to_dev(packed))
    S, Z = to_dev(s, BF16), to_dev(z, BF16)
    ids = ids_for(vocab, 64, 3)
    rows = qg.embed_w4(to_dev(ids), tiled, S, Z, 64)
    W = qg.dequant_w4(tiled, S, Z, 64, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    valid = (ids >= 0) & (ids < vocab)
    got = rows.cpu()[torch.from_numpy(valid)]
    assert torch.equal(got, W.cpu()[torch.from_numpy(ids[valid]).long()])
    assert torch.count_nonzero(rows.cpu()[torch.from_numpy(~valid)]) == 0


def test_embed_w4_tied_vocab_table_full_size():
    # The decode workload's tied-vocab table (vocab 131072, hidden 2048,
    # group 64) and 2048 token ids, every row against the oracle.
    vocab, hidden, tokens = 131072, 2048, 2048
    packed, s, z, _ = si.w4_weights(vocab, hidden, 64, si.seed_of("cfg1", "w", vocab, hidden, 64))
    ids = ids_for(vocab, tokens, 11)
    tiled = qg.repack_w4(to_dev(packed))
    out = qg.embed_w4(to_dev(ids), tiled, to_dev(s, BF16), to_dev(z, BF16), 64)
    torch.cuda.synchronize()
    ref = oracle.embed4(ids, packed, s, z, 64, BF16)
    assert np.array_equal(to_bits(out), oracle.f32_to_bf16(ref))


def test_embed_leading_dims_and_empty():
    vocab, hidden = 32, 128
    packed, s, z, _ = si.w4_weights(vocab, hidden, 64, 5)
    tiled = qg.repack_w4(to_dev(packed))
    ids = np.array([[3, 4, 5], [31, 0, 1]], dtype=np.int32)
    out = qg.embed_w4(to_dev(ids), tiled, to_dev(s, BF16), to_dev(z, BF16), 64)
    torch.cuda.synchronize()
    assert out.shape == (2, 3, hidden)
    ref = oracle.embed4(ids.reshape(-1), packed, s, z, 64, BF16)
    assert np.array_equal(to_bits(out.reshape(6, hidden)), oracle.f32_to_bf16(ref))
    empty = qg.embed_w4(torch.empty(0, dtype=torch.int32, device="cuda"), tiled, to_dev(s, BF16),
                        to_dev(z, BF16), 64)
    assert empty.shape == (0, hidden)
