"""The C ABI without a GPU: the library loads, exports every function that
include/qgemm.h declares, and rejects invalid arguments on the host before
any HIP call (these calls never reach a kernel launch)."""
import ctypes
import os
import re

import numpy as np
import pytest

import weight_only_quantized_w8a16_amd as qg
from weight_only_quantized_w8a16_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qgemm.h")

OK, NULL, SHAPE, GROUP, DTYPE, ALIGN, WORKSPACE, UNSUP = 0, 1, 2, 3, 4, 5, 6, 7
FAKE = 0x100000          # 16-byte-aligned stand-in address; never dereferenced
BF16, FP16, FP32 = 1, 2, 3


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(q\w+)\s*\(", text)))


def test_header_and_binding_agree():
    assert sorted(_abi.SIGNATURES) == declared_functions()


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(_abi.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_version_and_strerror():
    L = qg.lib()
    assert L.qg_version() >= 10000
    for s in range(10):
        assert L.qg_strerror(s) != b"unknown status"
    assert L.qg_strerror(99) == b"unknown status"


def w4(**kw):
    a = dict(A=FAKE, B=FAKE, s=FAKE, z=FAKE, bias=None, C=FAKE, m=4, n=128, k=256, g=64, act=BF16,
             bdt=0, ws=None, wsb=0)
    a.update(kw)
    return qg.lib().qgemm_w4a16(a["A"], a["B"], a["s"], a["z"], a["bias"], a["C"], a["m"], a["n"],
                                a["k"], a["g"], a["act"], a["bdt"], a["ws"], a["wsb"], None)


def w8(**kw):
    a = dict(A=FAKE, B=FAKE, s=FAKE, bias=None, C=FAKE, m=4, n=128, k=256, g=-1, act=FP16, bdt=0)
    a.update(kw)
    return qg.lib().qgemm_w8a16(a["A"], a["B"], a["s"], a["bias"], a["C"], a["m"], a["n"], a["k"],
                                a["g"], a["act"], a["bdt"], None, 0, None)


@pytest.mark.parametrize("kw,status", [
    (dict(m=-1), SHAPE), (dict(n=-16), SHAPE), (dict(k=0), SHAPE),
    (dict(A=None), NULL), (dict(B=None), NULL), (dict(s=None), NULL),
    (dict(C=None), NULL), (dict(bdt=FP16), NULL),
    (dict(z=None, n=24), UNSUP),      # zeros are optional (scale-only int4)
    (dict(act=0), DTYPE), (dict(act=FP32), DTYPE), (dict(act=7), DTYPE),
    (dict(bias=FAKE, bdt=0), DTYPE), (dict(bias=FAKE, bdt=FP32), DTYPE),
    (dict(g=32), GROUP), (dict(g=-2), GROUP), (dict(g=512), GROUP), (dict(k=192, g=128), GROUP),
    (dict(g=-1, n=24), UNSUP), (dict(g=256, n=24), UNSUP),   # per channel: -1 or k
    (dict(n=24), UNSUP), (dict(k=192), UNSUP),
    (dict(A=FAKE + 8), ALIGN), (dict(B=FAKE + 4), ALIGN), (dict(C=FAKE + 2), ALIGN),
    (dict(s=FAKE + 1), ALIGN), (dict(z=FAKE + 1), ALIGN), (dict(bias=FAKE + 1, bdt=FP16), ALIGN),
    (dict(m=0), OK), (dict(n=0), OK),
])
def test_w4_validation(kw, status):
    assert w4(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(m=-2), SHAPE), (dict(k=-64), SHAPE),
    (dict(A=None), NULL), (dict(s=None), NULL), (dict(bdt=BF16), NULL),
    (dict(act=FP32), DTYPE), (dict(bias=FAKE, bdt=0), DTYPE),
    (dict(g=32), GROUP), (dict(g=256, k=512), GROUP), (dict(g=128, k=192), GROUP),
    (dict(g=0), GROUP),
    (dict(n=8), UNSUP), (dict(k=96, g=96), UNSUP),
    (dict(A=FAKE + 4), ALIGN), (dict(s=FAKE + 1), ALIGN),
    (dict(m=0), OK), (dict(g=256, m=0), OK),
])
def test_w8_validation(kw, status):
    assert w8(**kw) == status


def test_repack_and_dequant_validation():
    L = qg.lib()
    assert L.qrepack_w4(FAKE, FAKE, -16, 128, None) == SHAPE
    assert L.qrepack_w4(None, FAKE, 16, 128, None) == NULL
    assert L.qrepack_w4(FAKE, FAKE, 24, 128, None) == UNSUP
    assert L.qrepack_w4(FAKE, FAKE, 16, 64, None) == UNSUP
    assert L.qrepack_w4(FAKE + 4, FAKE, 16, 128, None) == ALIGN
    assert L.qrepack_w4(FAKE, FAKE, 0, 128, None) == OK
    assert L.qunrepack_w4(FAKE, None, 16, 128, None) == NULL
    assert L.qrepack_w8(FAKE, FAKE, 16, 96, None) == UNSUP
    assert L.qunrepack_w8(FAKE, FAKE, 16, 0, None) == OK
    for f in (L.qrepack_w8_kn, L.qunrepack_w8_kn):
        assert f(FAKE, FAKE, -16, 64, None) == SHAPE
        assert f(FAKE, None, 16, 64, None) == NULL
        assert f(FAKE, FAKE, 40, 64, None) == UNSUP
        assert f(FAKE, FAKE, 16, 96, None) == UNSUP
        assert f(FAKE, FAKE + 8, 16, 64, None) == ALIGN
        assert f(FAKE, FAKE, 0, 64, None) == OK
        assert f(FAKE, FAKE, 16, 64 * 65536, None) == UNSUP
    assert L.qdequant_w4(FAKE, FAKE, FAKE, FAKE, 16, 128, 32, BF16, FP32, None) == GROUP
    assert L.qdequant_w4(FAKE, FAKE, FAKE, FAKE, 16, 128, 64, BF16, FP16, None) == DTYPE
    assert L.qdequant_w4(FAKE, None, FAKE, FAKE, 16, 128, 64, BF16, FP32, None) == NULL
    assert L.qdequant_w4(FAKE, FAKE, None, FAKE, 24, 128, 64, BF16, FP32, None) == UNSUP   # no zeros: ok
    assert L.qdequant_w4(FAKE, FAKE, FAKE, FAKE, 24, 128, -1, BF16, FP32, None) == UNSUP   # per channel
    assert L.qdequant_w8(FAKE, FAKE, FAKE, 16, 128, 32, FP16, FP32, None) == GROUP
    assert L.qdequant_w8(FAKE, FAKE, FAKE, 16, 192, 128, FP16, FP32, None) == GROUP
    assert L.qdequant_w8(FAKE, FAKE, FAKE, 16, 128, -1, FP16, BF16, None) == DTYPE


def moe(**kw):
    a = dict(x=FAKE, lg=FAKE, w1=FAKE, s1=FAKE, z1=FAKE, w2=FAKE, s2=FAKE, z2=FAKE, out=FAKE, T=8,
             H=256, I=128, E=8, k=2, g=64, act=BF16, ids=None, w=None, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return qg.lib().qmoe_grouped(a["x"], a["lg"], a["w1"], a["s1"], a["z1"], a["w2"], a["s2"],
                                 a["z2"], a["out"], a["T"], a["H"], a["I"], a["E"], a["k"], a["g"],
                                 a["act"], a["ids"], a["w"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(T=-1), SHAPE), (dict(k=0), SHAPE), (dict(k=9), SHAPE), (dict(E=0), SHAPE),
    (dict(x=None), NULL), (dict(lg=None), NULL), (dict(z2=None), NULL),
    (dict(act=FP32), DTYPE), (dict(g=32), GROUP), (dict(I=96, g=64), GROUP),
    (dict(H=192), UNSUP), (dict(E=300, k=2), UNSUP), (dict(E=128, k=65), UNSUP),
    (dict(x=FAKE + 8), ALIGN), (dict(lg=FAKE + 2), ALIGN), (dict(ids=FAKE + 2), ALIGN),
    (dict(ws=None), WORKSPACE), (dict(wsb=1024), WORKSPACE), (dict(ws=FAKE + 16), ALIGN),
    (dict(T=0), OK),
])
def test_moe_validation(kw, status):
    assert moe(**kw) == status


def test_workspace_sizes():
    L = qg.lib()
    assert L.qgemm_workspace_size(1, 2048, 2048, 64, 4) == 0
    small = L.qmoe_workspace_size(16, 256, 128, 8, 2)
    big = L.qmoe_workspace_size(2048, 2048, 1408, 64, 6)
    # the fc1 activation and fc2 output intermediates dominate: R*(I + H)*2 bytes
    assert big >= 2048 * 6 * (1408 + 2048) * 2
    assert 0 < small < big
    assert L.qmoe_workspace_size(0, 256, 128, 8, 2) == 0


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(_abi, "LIB_PATH", str(tmp_path / "absent.so"))
    monkeypatch.setattr(_abi, "_lib", None)
    with pytest.raises(qg.QGemmError):
        _abi.lib()


def test_layout_helpers_are_permutations():
    from helpers import tiled_w4_expected, tiled_w8_expected
    p = np.random.default_rng(0).integers(0, 256, (32, 128), dtype=np.uint8)
    t = tiled_w4_expected(p)
    assert sorted(np.unpackbits(p).tolist()) == sorted(np.unpackbits(t).tolist())
    assert not np.array_equal(t, p)
    c = np.random.default_rng(1).integers(-128, 128, (16, 128)).astype(np.int8)
    t8 = tiled_w8_expected(c)
    assert sorted((t8.view(np.uint8) ^ 0x80).ravel().tolist()) == sorted(c.view(np.uint8).ravel().tolist())


def q4(**kw):
    a = dict(W=FAKE, p=FAKE, s=FAKE, z=FAKE, n=32, k=256, g=64, wdt=BF16, sdt=BF16)
    a.update(kw)
    return qg.lib().qquantize_w4(a["W"], a["p"], a["s"], a["z"], a["n"], a["k"], a["g"], a["wdt"],
                                 a["sdt"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(n=-1), SHAPE), (dict(k=-128), SHAPE),
    (dict(W=None), NULL), (dict(p=None), NULL), (dict(s=None), NULL), (dict(z=None), NULL),
    (dict(wdt=0), DTYPE), (dict(wdt=7), DTYPE), (dict(sdt=0), DTYPE), (dict(sdt=9), DTYPE),
    (dict(g=32), GROUP), (dict(g=-1), GROUP), (dict(k=192, g=128), GROUP), (dict(k=100), GROUP),
    (dict(W=FAKE + 8), ALIGN), (dict(p=FAKE + 4), ALIGN), (dict(s=FAKE + 1), ALIGN),
    (dict(sdt=FP32, z=FAKE + 2), ALIGN),
    (dict(n=0), OK), (dict(k=0), OK), (dict(n=0, W=None), OK),
])
def test_quantize_validation(kw, status):
    assert q4(**kw) == status


def test_workspace_query_and_alignment():
    L = qg.lib()
    # split-K partials: fp32 [m, n] slices where the plan splits K -- two on
    # the fused 64 x 64 tile (int4 here); int8 per channel at up to 128 rows
    # with few 64 x 128 code-converting tiles: about one workgroup per CU
    # (256 CUs assumed without a device), slices of a multiple of 8 steps
    # (K = 3584: 56 steps; m = 128: 56 tiles, four slices of 16, 16, 16, 8;
    # m = 64: 28 tiles, seven slices of 8)
    assert L.qgemm_workspace_size(128, 3072, 2048, 64, 4) == 2 * 128 * 3072 * 4
    assert L.qgemm_workspace_size(128, 3584, 3584, -1, 8) == 4 * 128 * 3584 * 4
    assert L.qgemm_workspace_size(64, 3584, 3584, -1, 8) == 7 * 64 * 3584 * 4
    # dequantize-then-dense: the whole weight in the activation type, n * k * 2
    # bytes, at 512 .. 1024 rows with few 256 x 256 tiles (256 CUs assumed
    # without a device)
    for args in [(512, 3072, 2048, 64, 4), (1024, 3072, 2048, 128, 4), (512, 4096, 2048, -1, 4),
                 (1024, 2048, 2048, 64, 4), (700, 3584, 3584, 64, 8), (1024, 3584, 3584, 128, 8)]:
        assert L.qgemm_workspace_size(*args) == args[1] * args[2] * 2, args
    # int8 per channel at those sizes: the tiles that convert codes after the
    # LDS read, no workspace
    for args in [(700, 3584, 3584, -1, 8), (1024, 3584, 3584, -1, 8), (512, 3584, 3584, -1, 8)]:
        assert L.qgemm_workspace_size(*args) == 0, args
    for args in [(511, 3072, 2048, 64, 4), (1025, 3072, 2048, 64, 4), (512, 2048, 2048, 64, 4),
                 (512, 13312, 2048, 64, 4), (1024, 18944, 3584, -1, 8), (256, 3584, 3584, -1, 8),
                 (16, 3072, 2048, 64, 4), (128, 131072, 2048, 64, 4),
                 (128, 18944, 3584, -1, 8),
                 (0, 3072, 2048, 64, 4), (128, 3072, 2048, 64, 5), (128, 3072, 2048, 96, 4)]:
        assert L.qgemm_workspace_size(*args) == 0, args
    # a workspace that is given must be 256-byte aligned (checked before any launch)
    assert w4(m=128, n=3072, k=2048, ws=FAKE + 16, wsb=1 << 20) == ALIGN


# -- W8A8 -----------------------------------------------------------------------

MODE = 9


def w8a8(**kw):
    a = dict(A=FAKE, B=FAKE, mode=3, ac=FAKE, ar=FAKE, C=FAKE, m=4, n=128, k=256, out=FP16,
             ws=None, wsb=0)
    a.update(kw)
    return qg.lib().qgemm_w8a8(a["A"], a["B"], a["mode"], a["ac"], a["ar"], a["C"], a["m"], a["n"],
                               a["k"], a["out"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(m=-1), SHAPE), (dict(n=-16), SHAPE), (dict(k=0), SHAPE),
    (dict(A=None), NULL), (dict(B=None), NULL), (dict(ac=None), NULL), (dict(ar=None), NULL),
    (dict(C=None), NULL),
    (dict(out=0), DTYPE), (dict(out=7), DTYPE),
    (dict(mode=4), MODE), (dict(mode=-1), MODE),
    (dict(n=24), UNSUP), (dict(k=192), UNSUP), (dict(k=131136), UNSUP),
    (dict(m=1 << 14, k=131072), UNSUP),
    (dict(A=FAKE + 8), ALIGN), (dict(B=FAKE + 4), ALIGN), (dict(C=FAKE + 2), ALIGN),
    (dict(ac=FAKE + 2), ALIGN), (dict(ar=FAKE + 1), ALIGN), (dict(ws=FAKE + 16, wsb=64), ALIGN),
    (dict(m=0), OK), (dict(n=0), OK), (dict(m=0, A=None), OK),
])
def test_w8a8_validation(kw, status):
    assert w8a8(**kw) == status


def test_w8a8_modes_and_workspace_query():
    # The four modes are 0..3 (weights per channel = 1, activations per
    # token = 2); a problem with few tiles asks for split-K partials, decode
    # (m <= 16) and large problems for none, invalid sizes for none.
    L = qg.lib()
    assert (_abi.QG_W8A8_PER_TENSOR, _abi.QG_W8A8_PER_CHANNEL, _abi.QG_W8A8_PER_TOKEN) == (0, 1, 2)
    assert L.qgemm_w8a8_workspace_size(64, 3584, 3584) > 0
    assert L.qgemm_w8a8_workspace_size(64, 3584, 3584) % 256 == 0
    assert L.qgemm_w8a8_workspace_size(1, 3584, 3584) == 0     # streaming decode kernel
    assert L.qgemm_w8a8_workspace_size(4096, 18944, 3584) == 0
    assert L.qgemm_w8a8_workspace_size(0, 3584, 3584) == 0
    assert L.qgemm_w8a8_workspace_size(1, 3584, 3500) == 0


# -- embedding lookup ---------------------------------------------------------------

def emb4(**kw):
    a = dict(ids=FAKE, T=8, tab=FAKE, layout=1, s=FAKE, z=FAKE, out=FAKE, vocab=256, hidden=256,
             g=64, act=BF16, odt=BF16)
    a.update(kw)
    return qg.lib().qembed_w4(a["ids"], a["T"], a["tab"], a["layout"], a["s"], a["z"], a["out"],
                              a["vocab"], a["hidden"], a["g"], a["act"], a["odt"], None)


def emb8(**kw):
    a = dict(ids=FAKE, T=8, tab=FAKE, layout=1, s=FAKE, out=FAKE, vocab=256, hidden=256, g=-1,
             act=FP16, odt=FP32)
    a.update(kw)
    return qg.lib().qembed_w8(a["ids"], a["T"], a["tab"], a["layout"], a["s"], a["out"], a["vocab"],
                              a["hidden"], a["g"], a["act"], a["odt"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(T=-1), SHAPE), (dict(vocab=0), SHAPE), (dict(hidden=0), SHAPE),
    (dict(ids=None), NULL), (dict(tab=None), NULL), (dict(s=None), NULL), (dict(out=None), NULL),
    (dict(act=FP32), DTYPE), (dict(odt=FP16), DTYPE), (dict(odt=0), DTYPE),
    (dict(layout=2), 9), (dict(layout=-1), 9),
    (dict(g=32), GROUP), (dict(hidden=320, g=128), GROUP),
    (dict(vocab=24), UNSUP), (dict(hidden=192, g=64), UNSUP), (dict(layout=0, hidden=36, g=-1), UNSUP),
    (dict(ids=FAKE + 2), ALIGN), (dict(tab=FAKE + 8), ALIGN), (dict(out=FAKE + 4), ALIGN),
    (dict(s=FAKE + 1), ALIGN), (dict(z=FAKE + 1), ALIGN),
    (dict(T=0), OK), (dict(T=0, ids=None), OK),
])
def test_embed_w4_validation(kw, status):
    assert emb4(**kw) == status


def test_embed_w4_zeros_optional_and_portable_multiples():
    # zeros may be NULL (scale-only); the portable layout needs only
    # hidden % 8 and no vocab multiple -- both stop at the (later) alignment
    # check when the out pointer is misaligned, proving they passed the rest.
    assert emb4(z=None, out=FAKE + 4) == ALIGN
    assert emb4(layout=0, vocab=7, hidden=136, g=-1, out=FAKE + 4) == ALIGN


@pytest.mark.parametrize("kw,status", [
    (dict(T=-3), SHAPE), (dict(s=None), NULL), (dict(act=0), DTYPE), (dict(layout=5), 9),
    (dict(g=96), GROUP), (dict(vocab=24), UNSUP), (dict(hidden=96, g=-1), UNSUP),
    (dict(tab=FAKE + 4), ALIGN), (dict(T=0), OK),
])
def test_embed_w8_validation(kw, status):
    assert emb8(**kw) == status


# -- MoE with the optional parts ------------------------------------------------------

def moe_ex(**kw):
    a = dict(x=FAKE, lg=FAKE, sel=None, fin=None, w1=FAKE, s1=FAKE, z1=FAKE, b1=None, w2=FAKE,
             s2=FAKE, z2=FAKE, b2=None, out=FAKE, T=8, H=128, I=128, E=4, k=2, g=64, norm=1,
             act=BF16, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return qg.lib().qmoe_grouped_ex(a["x"], a["lg"], a["sel"], a["fin"], a["w1"], a["s1"], a["z1"],
                                    a["b1"], a["w2"], a["s2"], a["z2"], a["b2"], a["out"], a["T"],
                                    a["H"], a["I"], a["E"], a["k"], a["g"], a["norm"], a["act"],
                                    None, None, a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(T=-1), SHAPE), (dict(k=5), SHAPE), (dict(x=None), NULL), (dict(act=FP32), DTYPE),
    (dict(norm=2), 9), (dict(norm=-1), 9), (dict(g=32), GROUP), (dict(H=192, g=64), UNSUP),
    (dict(sel=FAKE + 2), ALIGN), (dict(b1=FAKE + 8), ALIGN), (dict(b2=FAKE + 2), ALIGN),
    (dict(ws=None), WORKSPACE), (dict(wsb=16), WORKSPACE), (dict(T=0), OK),
])
def test_moe_ex_validation(kw, status):
    assert moe_ex(**kw) == status


def test_read_probe_validation_and_blocks():
    L = qg.lib()
    assert L.qg_read_probe(FAKE, 24, FAKE, None) == SHAPE
    assert L.qg_read_probe(None, 16, FAKE, None) == NULL
    assert L.qg_read_probe(FAKE, 16, None, None) == NULL
    assert L.qg_read_probe(FAKE + 8, 16, FAKE, None) == ALIGN
    assert L.qg_read_probe(FAKE, 16, FAKE + 2, None) == ALIGN
    assert L.qg_read_probe_blocks(0) == 1
    assert L.qg_read_probe_blocks(1 << 30) == (1 << 30) // (16 * 512 * 2)   # one pass: 512 threads x 2 pieces


def test_lds_probe_validation():
    L = qg.lib()
    assert L.qg_lds_probe(8, 4096, 0, FAKE, None) == SHAPE
    assert L.qg_lds_probe(8, 4096, 65537, FAKE, None) == SHAPE
    assert L.qg_lds_probe(8, 4, 256, FAKE, None) == SHAPE
    assert L.qg_lds_probe(8, 4100, 256, FAKE, None) == SHAPE
    assert L.qg_lds_probe(6, 4096, 256, FAKE, None) == MODE
    assert L.qg_lds_probe(8, 4096, 256, None, None) == NULL
    assert L.qg_lds_probe(8, 4096, 256, FAKE + 4, None) == ALIGN


# -- the torch binding refuses wrong shapes and dtypes before any pointer is
# passed (host tensors suffice: the checks run before the device checks) -----

import torch  # noqa: E402

BF, F16 = torch.bfloat16, torch.float16


def _t(shape, dtype):
    return torch.zeros(shape, dtype=dtype)


def _status(fn, *a, **kw):
    with pytest.raises(qg.QGemmError) as e:
        fn(*a, **kw)
    return e.value.status


def _w4_args(m=4, n=128, k=256, g=64, dt=BF):
    return dict(A=_t((m, k), dt), B_tiled=_t((n, k // 2), torch.uint8),
                scales=_t((n, k // g), dt), zeros=_t((n, k // g), dt))


@pytest.mark.parametrize("change,status", [
    (dict(A=_t((4, 256), torch.float32)), DTYPE),
    (dict(B_tiled=_t((128, 128), torch.int8)), DTYPE),
    (dict(B_tiled=_t((128, 64), torch.uint8)), SHAPE),            # k / 2 wrong
    (dict(scales=_t((128, 4), torch.float32)), DTYPE),           # fp32 scales, bf16 A
    (dict(scales=_t((128, 4), F16)), DTYPE),
    (dict(scales=_t((4, 128), BF)), SHAPE),                       # transposed
    (dict(scales=_t((128, 2), BF)), SHAPE),
    (dict(zeros=_t((128, 4), F16)), DTYPE),
    (dict(zeros=_t((128, 8), BF)), SHAPE),
    (dict(bias=_t((127,), F16)), SHAPE),
    (dict(bias=_t((128,), torch.float32)), DTYPE),
    (dict(out=_t((4, 127), BF)), SHAPE),
    (dict(out=_t((4, 128), F16)), DTYPE),
])
def test_binding_w4_rejects_bad_operands(change, status):
    a = _w4_args()
    a.update(change)
    assert _status(qg.gemm_w4a16, group_size=64, **a) == status


def test_binding_w4_per_channel_scale_shape():
    a = _w4_args(g=256)
    a["scales"], a["zeros"] = _t((128, 2), BF), _t((128,), BF)
    assert _status(qg.gemm_w4a16, group_size=-1, **a) == SHAPE


@pytest.mark.parametrize("change,status", [
    (dict(B_tiled=_t((128, 256), torch.uint8)), DTYPE),
    (dict(B_tiled=_t((128, 128), torch.int8)), SHAPE),
    (dict(scales=_t((128,), BF)), DTYPE),
    (dict(scales=_t((64,), F16)), SHAPE),
    (dict(scales=_t((128, 2), F16)), SHAPE),                      # group -1 needs [n]
    (dict(out=_t((4, 64), F16)), SHAPE),
])
def test_binding_w8_rejects_bad_operands(change, status):
    a = dict(A=_t((4, 256), F16), B_tiled=_t((128, 256), torch.int8), scales=_t((128,), F16))
    a.update(change)
    assert _status(qg.gemm_w8a16, group_size=-1, **a) == status


def test_binding_w8_group_scale_shape():
    a = dict(A=_t((4, 256), F16), B_tiled=_t((128, 256), torch.int8), scales=_t((2, 128), F16))
    assert _status(qg.gemm_w8a16, group_size=128, **a) == SHAPE


def _moe_args(T=8, H=128, I=128, E=4, g=64, dt=BF):
    return dict(x=_t((T, H), dt), logits=_t((T, E), torch.float32),
                w1_tiled=_t((E, 2 * I, H // 2), torch.uint8), s1=_t((E, 2 * I, H // g), dt),
                z1=_t((E, 2 * I, H // g), dt), w2_tiled=_t((E, H, I // 2), torch.uint8),
                s2=_t((E, H, I // g), dt), z2=_t((E, H, I // g), dt))


@pytest.mark.parametrize("change,status", [
    (dict(logits=_t((8, 4), BF)), DTYPE),
    (dict(logits=_t((7, 4), torch.float32)), SHAPE),
    (dict(w1_tiled=_t((4, 256, 32), torch.uint8)), SHAPE),
    (dict(w1_tiled=_t((3, 256, 64), torch.uint8)), SHAPE),
    (dict(w2_tiled=_t((4, 128, 32), torch.uint8)), SHAPE),
    (dict(s1=_t((4, 256, 2), torch.float32)), DTYPE),
    (dict(s1=_t((4, 2, 256), BF)), SHAPE),
    (dict(z2=_t((4, 128, 3), BF)), SHAPE),
    (dict(b1=_t((4, 128), BF)), SHAPE),
    (dict(b2=_t((4, 128), F16)), SHAPE),
    (dict(sel_logits=_t((8, 5), torch.float32)), SHAPE),
    (dict(finished=_t((7,), torch.bool)), SHAPE),
    (dict(topk=5), SHAPE),
])
def test_binding_moe_rejects_bad_operands(change, status):
    a = _moe_args()
    a["topk"] = 2
    a.update(change)
    assert _status(qg.moe_grouped, **a) == status


@pytest.mark.parametrize("call,status", [
    (lambda: qg.dequant_w4(_t((16, 64), torch.uint8), _t((16, 2), torch.float32), None, 64), DTYPE),
    (lambda: qg.dequant_w4(_t((16, 64), torch.uint8), _t((2, 16), BF), None, 64), SHAPE),
    (lambda: qg.dequant_w4(_t((16, 64), torch.uint8), _t((16, 2), BF), _t((16, 2), F16), 64), DTYPE),
    (lambda: qg.dequant_w4(_t((16, 64), torch.uint8), _t((16, 2), BF), None, 64, F16), DTYPE),
    (lambda: qg.dequant_w8(_t((16, 128), torch.int8), _t((16, 2), F16), torch.float32, -1), SHAPE),
    (lambda: qg.dequant_w8(_t((16, 128), torch.uint8), _t((16,), F16)), DTYPE),
    (lambda: qg.embed_w4(_t((3,), torch.int64), _t((16, 64), torch.uint8), _t((16, 2), BF), None, 64), DTYPE),
    (lambda: qg.embed_w4(_t((3,), torch.int32), _t((16, 64), torch.uint8), _t((16, 4), BF), None, 64), SHAPE),
    (lambda: qg.embed_w8(_t((3,), torch.int32), _t((16, 128), torch.int8), _t((8,), F16)), SHAPE),
    (lambda: qg.repack_w4(_t((16, 64), torch.int8)), DTYPE),
    (lambda: qg.repack_w8(_t((16, 64), torch.uint8)), DTYPE),
    (lambda: qg.quantize_w4(_t((16, 128), torch.int32)), DTYPE),
    (lambda: qg.gemm_w8a8(_t((4, 128), torch.int8), _t((16, 64), torch.int8), _t((1,), torch.float32),
                          _t((1,), torch.float32)), SHAPE),
    (lambda: qg.gemm_w8a8(_t((4, 128), torch.int8), _t((16, 128), torch.int8), _t((1,), F16),
                          _t((1,), torch.float32)), DTYPE),
])
def test_binding_other_calls_reject_bad_operands(call, status):
    assert _status(call) == status


def test_binding_device_check_follows_shape_checks():
    # Right shapes and dtypes on the host: the device check is what refuses.
    assert _status(qg.gemm_w4a16, group_size=64, **_w4_args()) == NULL


def test_override_spec_validation():
    L = qg.lib()
    assert L.qg_set_override(b"path=decode,prefill_tile=D8,splitk=2,moe_tile=S,"
                             b"w8a8_tile=T64,w8a8_split=3") == OK
    for bad in (b"path=fast", b"tile=D8", b"splitk=0", b"prefill_tile=Q", b"w8a8_tile=7",
                b"moe_tile=L", b"splitk", b"splitk=2x"):
        assert L.qg_set_override(bad) == 9, bad
    assert L.qg_set_override(None) == OK and L.qg_set_override(b"") == OK
    qg.set_override(path="prefill")
    qg.set_override(splitk=3)
    assert qg._override == {"path": "prefill", "splitk": 3}
    qg.set_override(path=None)
    assert qg._override == {"splitk": 3}
    qg.clear_override()
    assert qg._override == {}


def test_moe_noalloc_rejects_problems_beyond_the_scratch():
    # 2048 tokens at hidden 2048, inter 1408, 64 experts, top-6 need ~81 MiB
    # of workspace (> the 64 MiB device scratch): refused on the host, before
    # any pointer is touched.
    L = qg.lib()
    assert L.qmoe_workspace_size(2048, 2048, 1408, 64, 6) > (64 << 20)
    args = [FAKE] * 9
    assert L.qmoe_grouped_noalloc(*args, 2048, 2048, 1408, 64, 6, 64, BF16, None, None, None) == WORKSPACE
    assert L.qmoe_grouped_noalloc(*args, 0, 2048, 1408, 64, 6, 64, BF16, None, None, None) == OK
    assert L.qmoe_grouped_noalloc(*args, 64, 2048, 1408, 64, 7, 32, BF16, None, None, None) == GROUP
