"""ctypes front end of the CPU oracle (``pkv_oracle.c``).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  Nothing here is imported by the GPU
library or its Python binding, and nothing here imports them.

All arrays are numpy arrays on the host.  bf16 data travels as ``uint16``
bit patterns.  The cache arrays follow the layout the oracle documents:
K ``[NB, Hkv, BS, D]``, V ``[NB, Hkv, BS/16, D, 16]`` (pages of channel-major 16-slot tiles), scales
``[NB, Hkv, BS]`` (per token), ``[NB, Hkv]`` (per block) or ``[Hkv, D]`` (static per channel).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pkv_oracle.c")
_LIB = os.path.join(_HERE, "libpkv_oracle.so")

# Plain IEEE arithmetic: no FMA contraction, no fast-math, default rounding.
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
          "-pthread", "-Wall", "-Wextra", "-Wno-unused-parameter"]


def build(force: bool = True) -> str:
    """Compile ``pkv_oracle.c`` with gcc into ``libpkv_oracle.so``."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.run(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        path = os.environ.get("PKV_ORACLE_LIB")  # a differently built copy (e.g. with AddressSanitizer)
        if not path:
            build(force=False)
            path = _LIB
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        I = ctypes.c_int
        L.oracle_bf16_round.argtypes = [ctypes.c_double]
        L.oracle_bf16_round.restype = ctypes.c_uint16
        L.oracle_store.argtypes = [I, I, I, I, I, P, P, P, P, P, P, I, P, P, P, P, I, I]
        L.oracle_store.restype = I
        L.oracle_dequant.argtypes = [I, I, I, I, I, P, P, P, P, P, I, P, P, I, P, P,
                                     ctypes.c_int64, ctypes.c_int64]
        L.oracle_dequant.restype = I
        L.oracle_decode.argtypes = [I, I, I, I, I, P, P, P, P, P, I, P, I, P, P, I,
                                    ctypes.c_double, P, P, P, I, I]
        L.oracle_decode.restype = I
        L.oracle_mla_store.argtypes = [I, I, I, I, P, P, P, P, P, P, I, P, P, P, P, I, I]
        L.oracle_mla_store.restype = I
        L.oracle_mla_decode.argtypes = [I, I, I, I, P, P, P, P, P, P, I, P, I, P, I,
                                        ctypes.c_double, P, P, P, I]
        L.oracle_mla_decode.restype = I
        _lib = L
    return _lib


def _p(a):
    if a is None:
        return None
    if not a.flags["C_CONTIGUOUS"]:
        raise ValueError("oracle arrays must be C-contiguous")
    return a.ctypes.data


def _check(arr, dtype, name):
    if arr is not None and arr.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {arr.dtype}")


class HostCache:
    """A host copy of a paged cache in the contract layout."""

    def __init__(self, mode, num_blocks, num_kv_heads, block_size, head_dim, fill=0):
        self.mode, self.nb, self.hkv, self.bs, self.d = mode, num_blocks, num_kv_heads, block_size, head_dim
        dt = np.uint16 if mode == 2 else np.int8
        self.k = np.full((num_blocks, num_kv_heads, block_size, head_dim), fill, dtype=dt)
        vt = 16 if block_size % 16 == 0 else block_size  # slots per V tile
        self.v = np.full((num_blocks, num_kv_heads, block_size // vt, head_dim, vt), fill, dtype=dt)
        if mode == 0:
            self.k_scale = np.zeros((num_blocks, num_kv_heads, block_size), np.float32)
            self.v_scale = np.zeros((num_blocks, num_kv_heads, block_size), np.float32)
        elif mode == 1:
            self.k_scale = np.zeros((num_blocks, num_kv_heads), np.float32)
            self.v_scale = np.zeros((num_blocks, num_kv_heads), np.float32)
        elif mode == 3:  # static per-channel scales: inputs, set by the caller
            self.k_scale = np.zeros((num_kv_heads, head_dim), np.float32)
            self.v_scale = np.zeros((num_kv_heads, head_dim), np.float32)
        else:
            self.k_scale = self.v_scale = None

    def args(self):
        return (self.mode, self.nb, self.hkv, self.bs, self.d, _p(self.k), _p(self.v),
                _p(self.k_scale), _p(self.v_scale))

    def copy(self):
        c = HostCache.__new__(HostCache)
        c.__dict__.update(self.__dict__)
        c.k, c.v = self.k.copy(), self.v.copy()
        c.k_scale = None if self.k_scale is None else self.k_scale.copy()
        c.v_scale = None if self.v_scale is None else self.v_scale.copy()
        return c


def bf16_round(x: float) -> int:
    """Bit pattern of the bf16 nearest to ``x`` (ties to even)."""
    return int(lib().oracle_bf16_round(float(x)))


def store(cache: HostCache, k_new, v_new, *, slot_mapping=None, cu_q_lens=None,
          context_lengths=None, block_table=None):
    """Quantize and write new tokens (bf16 bits ``uint16 [T, Hkv, D]``) into ``cache``."""
    _check(k_new, np.uint16, "k_new")
    _check(v_new, np.uint16, "v_new")
    k_new = np.ascontiguousarray(k_new)
    v_new = np.ascontiguousarray(v_new)
    t = k_new.shape[0]
    sm = None if slot_mapping is None else np.ascontiguousarray(slot_mapping, np.int64)
    cu = None if cu_q_lens is None else np.ascontiguousarray(cu_q_lens, np.int32)
    ctx = None if context_lengths is None else np.ascontiguousarray(context_lengths, np.int32)
    bt = None if block_table is None else np.ascontiguousarray(block_table, np.int32)
    batch = 0 if ctx is None else len(ctx)
    mbs = 0 if bt is None else bt.shape[1]
    rc = lib().oracle_store(*cache.args(), _p(k_new), _p(v_new), t, _p(sm), _p(cu), _p(ctx),
                            _p(bt), batch, mbs)
    if rc != 0:
        raise ValueError("oracle_store rejected its arguments")


def dequant(cache: HostCache, block_table, context_lengths, *, seq_offsets=None, out_rows=None,
            k_out=None, v_out=None, token_stride=None, head_stride=None):
    """Gather the cache back to bf16 bits. Returns (k_out, v_out) ``uint16``."""
    bt = np.ascontiguousarray(block_table, np.int32)
    ctx = np.ascontiguousarray(context_lengths, np.int32)
    so = None if seq_offsets is None else np.ascontiguousarray(seq_offsets, np.int64)
    if out_rows is None:
        out_rows = int(ctx.sum()) if so is None else int((so + ctx).max(initial=0))
    if token_stride is None:
        token_stride = cache.hkv * cache.d
    if head_stride is None:
        head_stride = cache.d
    if k_out is None:
        k_out = np.zeros(max(out_rows * token_stride, 1), np.uint16)
    if v_out is None:
        v_out = np.zeros(max(out_rows * token_stride, 1), np.uint16)
    rc = lib().oracle_dequant(*cache.args(), _p(bt), bt.shape[1], _p(ctx), _p(so), len(ctx),
                              _p(k_out), _p(v_out), int(token_stride), int(head_stride))
    if rc != 0:
        raise ValueError("oracle_dequant rejected its arguments")
    return k_out, v_out


def decode(cache: HostCache, q, num_q_heads, block_table, context_lengths, scale, *,
           cu_q_lens=None, nthreads=1, want_f64=True, window=0):
    """fp64 attention. ``q``: bf16 bits ``uint16 [Tq, Hq, D]``; ``window`` > 0 limits each query to
    its last ``window`` keys (itself included).

    Returns (out_bf16 uint16 [Tq, Hq, D], out_f64 or None, lse fp64 [Tq, Hq]).
    """
    _check(q, np.uint16, "q")
    q = np.ascontiguousarray(q)
    bt = np.ascontiguousarray(block_table, np.int32)
    ctx = np.ascontiguousarray(context_lengths, np.int32)
    cu = None if cu_q_lens is None else np.ascontiguousarray(cu_q_lens, np.int32)
    tq = q.shape[0]
    out = np.zeros((tq, num_q_heads, cache.d), np.uint16)
    out64 = np.zeros((tq, num_q_heads, cache.d), np.float64) if want_f64 else None
    lse = np.zeros((tq, num_q_heads), np.float64)
    rc = lib().oracle_decode(*cache.args(), _p(q), num_q_heads, _p(bt), bt.shape[1], _p(ctx),
                             _p(cu), len(ctx), float(scale), _p(out), _p(out64), _p(lse),
                             int(nthreads), int(window))
    if rc != 0:
        raise ValueError("oracle_decode rejected its arguments")
    return out, out64, lse


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Reinterpret bf16 bit patterns as fp32 values (exact)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


class MLAHostCache:
    """A host copy of a paged MLA cache: latent codes ``int8 [NB, BS, Dc]``, rotary-key codes
    ``int8 [NB, BS, Dr]``, and one fp32 scale per token for each, ``[NB, BS]``."""

    def __init__(self, num_blocks, block_size, latent_dim, rope_dim):
        self.nb, self.bs, self.dc, self.dr = num_blocks, block_size, latent_dim, rope_dim
        self.latent = np.zeros((num_blocks, block_size, latent_dim), np.int8)
        self.rope = np.zeros((num_blocks, block_size, rope_dim), np.int8)
        self.latent_scale = np.zeros((num_blocks, block_size), np.float32)
        self.rope_scale = np.zeros((num_blocks, block_size), np.float32)

    def args(self):
        return (self.nb, self.bs, self.dc, self.dr, _p(self.latent), _p(self.rope),
                _p(self.latent_scale), _p(self.rope_scale))

    def copy(self):
        c = MLAHostCache.__new__(MLAHostCache)
        c.__dict__.update(self.__dict__)
        for k in ("latent", "rope", "latent_scale", "rope_scale"):
            setattr(c, k, getattr(self, k).copy())
        return c


def mla_store(cache: MLAHostCache, latent_new, rope_new, *, slot_mapping=None, cu_q_lens=None,
              context_lengths=None, block_table=None):
    """Quantize and write new tokens (bf16 bits ``uint16 [T, Dc]`` and ``[T, Dr]``)."""
    _check(latent_new, np.uint16, "latent_new")
    _check(rope_new, np.uint16, "rope_new")
    latent_new = np.ascontiguousarray(latent_new)
    rope_new = np.ascontiguousarray(rope_new)
    sm = None if slot_mapping is None else np.ascontiguousarray(slot_mapping, np.int64)
    cu = None if cu_q_lens is None else np.ascontiguousarray(cu_q_lens, np.int32)
    ctx = None if context_lengths is None else np.ascontiguousarray(context_lengths, np.int32)
    bt = None if block_table is None else np.ascontiguousarray(block_table, np.int32)
    batch = 0 if ctx is None else len(ctx)
    mbs = 0 if bt is None else bt.shape[1]
    rc = lib().oracle_mla_store(*cache.args(), _p(latent_new), _p(rope_new), latent_new.shape[0],
                                _p(sm), _p(cu), _p(ctx), _p(bt), batch, mbs)
    if rc != 0:
        raise ValueError("oracle_mla_store rejected its arguments")


def mla_decode(cache: MLAHostCache, q_latent, q_rope, block_table, context_lengths, scale, *,
               nthreads=1, want_f64=True):
    """fp64 latent attention of one query per sequence. ``q_latent``: bf16 bits ``[B, H, Dc]``,
    ``q_rope``: ``[B, H, Dr]``.  Returns (out_bf16 uint16 [B, H, Dc], out_f64 or None,
    lse fp64 [B, H])."""
    _check(q_latent, np.uint16, "q_latent")
    _check(q_rope, np.uint16, "q_rope")
    ql = np.ascontiguousarray(q_latent)
    qr = np.ascontiguousarray(q_rope)
    bt = np.ascontiguousarray(block_table, np.int32)
    ctx = np.ascontiguousarray(context_lengths, np.int32)
    b, h = ql.shape[0], ql.shape[1]
    out = np.zeros((b, h, cache.dc), np.uint16)
    out64 = np.zeros((b, h, cache.dc), np.float64) if want_f64 else None
    lse = np.zeros((b, h), np.float64)
    rc = lib().oracle_mla_decode(*cache.args(), _p(ql), _p(qr), h, _p(bt), bt.shape[1], _p(ctx),
                                 len(ctx), float(scale), _p(out), _p(out64), _p(lse), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_mla_decode rejected its arguments")
    return out, out64, lse
