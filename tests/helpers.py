"""Shared test helpers: bf16 bit handling, exact-rational rounding, tolerance checks.

Nothing here implements the method under test; the exact-rational routines are
independent re-derivations of IEEE rounding used to pin the oracle.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np


def torch_bf16_to_bits(t) -> np.ndarray:
    import torch

    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def bits_to_f32(bits) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_to_bits(x) -> np.ndarray:
    """fp32 -> bf16 bits by truncation; only for values already on the bf16 grid."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value not representable in bf16"
    return (u >> 16).astype(np.uint16)


def all_finite_bf16_bits() -> np.ndarray:
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    exp = (b >> 7) & 0xFF
    return b[exp != 0xFF]


def nearest_binary(fr: Fraction, mant_bits: int, min_exp: int) -> Fraction:
    """Exact nearest value on a binary floating-point grid (ties to even), no overflow."""
    if fr == 0:
        return Fraction(0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, min_exp)
    spacing = Fraction(2) ** (e - mant_bits)
    n = a / spacing
    lo = math.floor(n)
    rem = n - lo
    k = lo + 1 if (rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1)) else lo
    return sign * k * spacing


def nearest_f32(fr: Fraction) -> Fraction:
    return nearest_binary(fr, 23, -126)


def nearest_bf16(fr: Fraction) -> Fraction:
    return nearest_binary(fr, 7, -126)


def attention_close(gpu, ref64, atol=1e-2, rtol=1e-2):
    """Attention tolerance: max abs <= atol, norm-relative <= rtol, elementwise abs <= atol + rtol|ref|."""
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref64, dtype=np.float64)
    err = np.abs(g - r)
    max_abs = float(err.max(initial=0.0))
    denom = float(np.linalg.norm(r))
    rel = float(np.linalg.norm(g - r) / denom) if denom > 0 else float(np.linalg.norm(g - r))
    elem_ok = bool(np.all(err <= atol + rtol * np.abs(r)))
    return max_abs, rel, elem_ok


# ---- V page layout: [NB, Hkv, BS/T, D, T], tiles of T slots, each channel-major (T = 16 for
#      every block size the GPU library takes; the CPU oracle also takes block sizes that are not
#      multiples of 16, whose page is then one tile of T = BS slots)
def vtile(bs: int) -> int:
    return 16 if bs % 16 == 0 else bs


def v_slot(v, blk, h, off, bs):
    """The head_dim values of slot `off` of page (blk, h): a (writable) strided view."""
    t = vtile(bs)
    return v[blk, h, off // t, :, off % t]


def v_token_major(v, bs):
    """V pages rearranged to [NB, Hkv, BS, D] (numpy array or torch tensor, host)."""
    t = vtile(bs)
    nb, hkv = v.shape[0], v.shape[1]
    x = v.reshape(nb, hkv, bs // t, -1, t)
    x = x.transpose(0, 1, 2, 4, 3) if isinstance(x, np.ndarray) else x.permute(0, 1, 2, 4, 3)
    return x.reshape(nb, hkv, bs, -1)
