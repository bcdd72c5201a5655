"""Shared test helpers: moving seeded numpy bit patterns onto the GPU and
back, the relative-error metric, and the documented tiled layouts written as
numpy index arithmetic (to check the library's repack against its header)."""
import numpy as np
import torch

BF16, FP16 = 1, 2
TORCH_DT = {BF16: torch.bfloat16, FP16: torch.float16}
TOL = {BF16: 1e-2, FP16: 3e-3}   # max|C - Cref| / max|Cref|


def to_dev(bits, dtype=None, device="cuda"):
    """numpy array -> device tensor; uint16 bit patterns are viewed as dtype."""
    a = np.ascontiguousarray(bits)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16).copy()).view(TORCH_DT[dtype])
    else:
        t = torch.from_numpy(a.copy())
    return t.to(device)


def to_bits(t):
    """16-bit device/host tensor -> numpy uint16 bit patterns."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def rel_err(C, Cref):
    C = np.asarray(C, dtype=np.float64)
    Cref = np.asarray(Cref, dtype=np.float64)
    denom = np.abs(Cref).max()
    return float(np.abs(C - Cref).max() / (denom if denom > 0 else 1.0))


def widen(bits, dtype):
    """uint16 bit patterns -> float64 (exact), by torch's own widening."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).copy()).view(TORCH_DT[dtype])
    return t.double().numpy()


def tiled_w4_expected(packed):
    """Tiled int4 bytes for a portable [n, k/2] matrix, from the layout formula
    in include/qgemm.h."""
    n, half = packed.shape
    k = half * 2
    codes = np.empty((n, k), dtype=np.uint8)
    codes[:, 0::2] = packed & 0xF
    codes[:, 1::2] = packed >> 4
    nn, kk = np.meshgrid(np.arange(n), np.arange(k), indexing="ij")
    nt, nl, kb, r = nn // 16, nn % 16, kk // 128, kk % 128
    t, j, e = r // 32, (r // 8) % 4, kk % 8
    lane = 16 * j + nl
    pos = np.where(e % 2 == 0, e // 2, 4 + e // 2)
    byte = (nt * (k // 128) + kb) * 1024 + lane * 16 + t * 4 + pos // 2
    out = np.zeros(n * half, dtype=np.uint8)
    np.add.at(out, byte.ravel(), (codes << (4 * (pos % 2))).astype(np.uint8).ravel())
    return out.reshape(n, half)


def tiled_w8_expected(codes):
    """Tiled int8 bytes for a portable [n, k] int8 matrix, from the layout
    formula in include/qgemm.h (offset binary)."""
    n, k = codes.shape
    nn, kk = np.meshgrid(np.arange(n), np.arange(k), indexing="ij")
    nt, nl, kb, r = nn // 16, nn % 16, kk // 64, kk % 64
    t, j, e = r // 32, (r // 8) % 4, kk % 8
    byte = (nt * (k // 64) + kb) * 1024 + (16 * j + nl) * 16 + t * 8 + e
    out = np.zeros(n * k, dtype=np.uint8)
    out[byte.ravel()] = (codes.view(np.uint8) ^ 0x80).ravel()
    return out.reshape(n, k).view(np.int8)
