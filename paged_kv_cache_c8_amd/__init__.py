"""Python binding of libpkv (include/pkv.h): argument marshalling only.

Every step of the store / dequant / decode path runs in the HIP kernels of ``libpkv.so``; this
module passes device pointers (``tensor.data_ptr()``) and the current HIP stream, and raises
``PkvError`` on a non-zero status.  PyTorch supplies device memory and streams.

There is no fallback: if ``libpkv.so`` has not been built, ``lib()`` raises.
"""
from __future__ import annotations

import ctypes
import os

import torch  # loaded first: libpkv binds to the HIP runtime torch has already loaded

__all__ = ["PkvError", "Cache", "lib", "store_c8", "dequant", "decode_gqa", "decode_workspace_size",
           "decode_plan", "MLACache", "mla_store_c8", "mla_decode", "mla_decode_workspace_size",
           "mla_decode_plan", "QUANT_PER_TOKEN", "QUANT_PER_BLOCK", "QUANT_NONE_BF16", "QUANT_PER_CHANNEL",
           "EXPORTS"]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpkv.so")

QUANT_PER_TOKEN = 0
QUANT_PER_BLOCK = 1
QUANT_NONE_BF16 = 2
QUANT_PER_CHANNEL = 3

# every symbol include/pkv.h declares
EXPORTS = ("pkv_status_string", "pkv_version", "pkv_store_c8", "pkv_dequant",
           "pkv_decode_workspace_size", "pkv_decode_gqa", "pkv_decode_plan", "pkv_mla_store_c8",
           "pkv_mla_decode_workspace_size", "pkv_mla_decode_plan", "pkv_mla_decode")

MLA_LATENT_DIM = 512
MLA_ROPE_DIM = 64


class PkvError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {lib().pkv_status_string(status).decode()} ({status})")


class _CacheT(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("k_scale", ctypes.c_void_p),
                ("v_scale", ctypes.c_void_p), ("num_blocks", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("quant_mode", ctypes.c_int32)]


class _MLACacheT(ctypes.Structure):
    _fields_ = [("latent", ctypes.c_void_p), ("rope", ctypes.c_void_p), ("latent_scale", ctypes.c_void_p),
                ("rope_scale", ctypes.c_void_p), ("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("latent_dim", ctypes.c_int32), ("rope_dim", ctypes.c_int32)]


class _DecodeOpts(ctypes.Structure):
    _fields_ = [("split_tokens", ctypes.c_int32), ("kernel", ctypes.c_int32),
                ("partition", ctypes.c_int32), ("window", ctypes.c_int32), ("reserved", ctypes.c_int32 * 4)]


_lib = None


def lib():
    """The loaded libpkv.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m paged_kv_cache_c8_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        L.pkv_status_string.argtypes = [ctypes.c_int]
        L.pkv_status_string.restype = ctypes.c_char_p
        L.pkv_version.argtypes = []
        L.pkv_version.restype = ctypes.c_int
        L.pkv_store_c8.argtypes = [P, P, P, I32, P, P, P, P, I32, I32, I32, I32, P]
        L.pkv_store_c8.restype = ctypes.c_int
        L.pkv_dequant.argtypes = [P, P, I32, P, P, I32, P, P, I64, I64, P]
        L.pkv_dequant.restype = ctypes.c_int
        L.pkv_decode_workspace_size.argtypes = [I32, I32, I32, I32, I32, I32, I32, I32, P]
        L.pkv_decode_workspace_size.restype = SZ
        L.pkv_decode_gqa.argtypes = [P, I32, P, P, I32, P, P, I32, I32, ctypes.c_float, P, P, P, SZ,
                                     P, P]
        L.pkv_decode_gqa.restype = ctypes.c_int
        L.pkv_decode_plan.argtypes = [I32, I32, I32, I32, I32, I32, I32, I32, P,
                                      ctypes.POINTER(I32), ctypes.POINTER(I32), ctypes.POINTER(I32)]
        L.pkv_decode_plan.restype = ctypes.c_int
        L.pkv_mla_store_c8.argtypes = [P, P, P, I32, P, P, P, P, I32, I32, P]
        L.pkv_mla_store_c8.restype = ctypes.c_int
        L.pkv_mla_decode_workspace_size.argtypes = [I32, I32, I32, I32, I32]
        L.pkv_mla_decode_workspace_size.restype = SZ
        L.pkv_mla_decode_plan.argtypes = [I32, I32, I32, I32, I32, ctypes.POINTER(I32), ctypes.POINTER(I32)]
        L.pkv_mla_decode_plan.restype = ctypes.c_int
        L.pkv_mla_decode.argtypes = [P, P, I32, P, P, I32, P, I32, ctypes.c_float, P, P, P, SZ, I32, P]
        L.pkv_mla_decode.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _check(status, what):
    if status != 0:
        raise PkvError(status, what)


PARTITION_PLANNED, PARTITION_FIXED, PARTITION_BALANCED = 0, 1, 2


def _opts(split_tokens=0, kernel=0, partition=0, window=0):
    o = _DecodeOpts()
    o.split_tokens = int(split_tokens)
    o.kernel = int(kernel)
    o.partition = int(partition)
    o.window = int(window)
    return o


class Cache:
    """A paged cache in device memory: K ``[NB, Hkv, BS, D]``, V ``[NB, Hkv, BS/16, D, 16]`` (pages
    of channel-major 16-slot tiles; int8, or bf16 in mode 2), scales ``[NB, Hkv, BS]`` (mode 0),
    ``[NB, Hkv]`` (mode 1) or ``[Hkv, D]`` (mode 3: static per-channel scales the caller sets)."""

    def __init__(self, quant_mode, num_blocks, num_kv_heads, block_size, head_dim, device="cuda",
                 k=None, v=None, k_scale=None, v_scale=None):
        self.quant_mode = int(quant_mode)
        self.num_blocks, self.num_kv_heads = int(num_blocks), int(num_kv_heads)
        self.block_size, self.head_dim = int(block_size), int(head_dim)
        dt = torch.bfloat16 if self.quant_mode == QUANT_NONE_BF16 else torch.int8
        shape_k = (num_blocks, num_kv_heads, block_size, head_dim)
        shape_v = (num_blocks, num_kv_heads, max(1, block_size // 16), head_dim, min(block_size, 16))
        self.k = k if k is not None else torch.zeros(shape_k, dtype=dt, device=device)
        self.v = v if v is not None else torch.zeros(shape_v, dtype=dt, device=device)
        if self.quant_mode == QUANT_PER_TOKEN:
            sshape = (num_blocks, num_kv_heads, block_size)
        elif self.quant_mode == QUANT_PER_BLOCK:
            sshape = (num_blocks, num_kv_heads)
        elif self.quant_mode == QUANT_PER_CHANNEL:
            sshape = (num_kv_heads, head_dim)
        else:
            sshape = None
        if sshape is None:
            self.k_scale = self.v_scale = None
        else:
            self.k_scale = k_scale if k_scale is not None else torch.zeros(sshape, dtype=torch.float32, device=device)
            self.v_scale = v_scale if v_scale is not None else torch.zeros(sshape, dtype=torch.float32, device=device)
        for t in (self.k, self.v, self.k_scale, self.v_scale):
            if t is not None and not t.is_contiguous():
                raise ValueError("cache tensors must be contiguous")
        self._c = _CacheT(self.k.data_ptr(), self.v.data_ptr(), _ptr(self.k_scale), _ptr(self.v_scale),
                          self.num_blocks, self.num_kv_heads, self.block_size, self.head_dim,
                          self.quant_mode)

    @property
    def ref(self):
        return ctypes.byref(self._c)


def store_c8(cache: Cache, k_new, v_new, *, slot_mapping=None, cu_q_lens=None, context_lengths=None,
             block_table=None, max_q_len=0, stream=None):
    """Quantize (or copy, mode 2) bf16 ``[T, Hkv, D]`` tokens into the cache."""
    t = int(k_new.shape[0])
    batch = 0 if context_lengths is None else int(context_lengths.shape[0])
    mbs = 0 if block_table is None else int(block_table.shape[1])
    st = lib().pkv_store_c8(cache.ref, _ptr(k_new), _ptr(v_new), t, _ptr(slot_mapping), _ptr(cu_q_lens),
                            _ptr(context_lengths), _ptr(block_table), batch, mbs, int(max_q_len),
                            cache.quant_mode, _stream(stream))
    _check(st, "pkv_store_c8")


def dequant(cache: Cache, block_table, context_lengths, *, seq_offsets=None, k_out=None, v_out=None,
            token_stride=None, head_stride=None, stream=None):
    """Gather to bf16 rows.  Default outputs: packed ``[sum(ctx), Hkv, D]`` tensors (this shape
    needs the context lengths on the host, which the call itself never reads)."""
    if k_out is None and v_out is None:
        rows = int(context_lengths.sum().item()) if seq_offsets is None else \
            int((seq_offsets + context_lengths.to(seq_offsets.dtype)).max().item())
        k_out = torch.empty((max(rows, 1), cache.num_kv_heads, cache.head_dim), dtype=torch.bfloat16,
                            device=cache.k.device)
        v_out = torch.empty_like(k_out)
    if token_stride is None:
        token_stride = cache.num_kv_heads * cache.head_dim
    if head_stride is None:
        head_stride = cache.head_dim
    st = lib().pkv_dequant(cache.ref, _ptr(block_table), int(block_table.shape[1]), _ptr(context_lengths),
                           _ptr(seq_offsets), int(context_lengths.shape[0]), _ptr(k_out), _ptr(v_out),
                           int(token_stride), int(head_stride), _stream(stream))
    _check(st, "pkv_dequant")
    return k_out, v_out


def decode_workspace_size(batch, num_q_heads, cache: Cache, max_blocks_per_seq, max_q_len=1,
                          split_tokens=0, kernel=0, partition=0, window=0) -> int:
    o = _opts(split_tokens, kernel, partition, window)
    return int(lib().pkv_decode_workspace_size(batch, num_q_heads, cache.num_kv_heads, cache.head_dim,
                                               max_blocks_per_seq, cache.block_size, max_q_len,
                                               cache.quant_mode, ctypes.byref(o)))


def decode_plan(batch, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq, block_size,
                max_q_len=1, quant_mode=0, split_tokens=0, kernel=0, partition=0, window=0):
    o = _opts(split_tokens, kernel, partition, window)
    a, b, c = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    st = lib().pkv_decode_plan(batch, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq, block_size,
                               max_q_len, quant_mode, ctypes.byref(o), ctypes.byref(a), ctypes.byref(b),
                               ctypes.byref(c))
    _check(st, "pkv_decode_plan")
    return {"split_tokens": a.value, "num_splits": b.value, "kernel": c.value}


def decode_gqa(q, cache: Cache, block_table, context_lengths, scale, *, cu_q_lens=None, max_q_len=1,
               out=None, lse_out=None, workspace=None, split_tokens=0, kernel=0, partition=0, window=0,
               stream=None):
    """Attention of the new queries ``q`` (bf16 ``[Tq, Hq, D]``) over the paged cache."""
    hq = int(q.shape[1])
    batch = int(context_lengths.shape[0])
    mbs = int(block_table.shape[1])
    if cu_q_lens is None:
        max_q_len = 1
    if out is None:
        out = torch.empty_like(q)
    o = _opts(split_tokens, kernel, partition, window)
    need = int(lib().pkv_decode_workspace_size(batch, hq, cache.num_kv_heads, cache.head_dim, mbs,
                                               cache.block_size, max_q_len, cache.quant_mode,
                                               ctypes.byref(o)))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)  # no initial contents needed
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().pkv_decode_gqa(_ptr(q), hq, cache.ref, _ptr(block_table), mbs, _ptr(context_lengths),
                              _ptr(cu_q_lens), batch, int(max_q_len), float(scale), _ptr(out),
                              _ptr(lse_out), _ptr(workspace), ws_bytes, ctypes.byref(o), _stream(stream))
    _check(st, "pkv_decode_gqa")
    return out


# ---------------------------------------------------------------------------------------------
# paged MLA (latent) cache
# ---------------------------------------------------------------------------------------------

class MLACache:
    """A paged latent cache in the layout include/pkv.h documents: ``latent`` int8
    ``[NB, BS, 512]``, ``rope`` int8 ``[NB, BS, 64]``, ``latent_scale`` / ``rope_scale`` fp32
    ``[NB, BS]`` (one per token)."""

    def __init__(self, num_blocks, block_size, device="cuda", latent_dim=MLA_LATENT_DIM, rope_dim=MLA_ROPE_DIM):
        self.num_blocks, self.block_size = int(num_blocks), int(block_size)
        self.latent_dim, self.rope_dim = int(latent_dim), int(rope_dim)
        self.latent = torch.zeros((num_blocks, block_size, latent_dim), dtype=torch.int8, device=device)
        self.rope = torch.zeros((num_blocks, block_size, rope_dim), dtype=torch.int8, device=device)
        self.latent_scale = torch.zeros((num_blocks, block_size), dtype=torch.float32, device=device)
        self.rope_scale = torch.zeros((num_blocks, block_size), dtype=torch.float32, device=device)
        self._c = _MLACacheT(self.latent.data_ptr(), self.rope.data_ptr(), self.latent_scale.data_ptr(),
                             self.rope_scale.data_ptr(), self.num_blocks, self.block_size, self.latent_dim,
                             self.rope_dim)

    @property
    def ref(self):
        return ctypes.byref(self._c)


def mla_store_c8(cache: MLACache, latent_new, rope_new, *, slot_mapping=None, cu_q_lens=None,
                 context_lengths=None, block_table=None, stream=None):
    """Quantize bf16 latent rows ``[T, 512]`` and rotary-key rows ``[T, 64]`` into the cache."""
    t = int(latent_new.shape[0])
    batch = 0 if context_lengths is None else int(context_lengths.shape[0])
    mbs = 0 if block_table is None else int(block_table.shape[1])
    st = lib().pkv_mla_store_c8(cache.ref, _ptr(latent_new), _ptr(rope_new), t, _ptr(slot_mapping),
                                _ptr(cu_q_lens), _ptr(context_lengths), _ptr(block_table), batch, mbs,
                                _stream(stream))
    _check(st, "pkv_mla_store_c8")


def mla_decode_workspace_size(batch, num_heads, max_blocks_per_seq, block_size, split_tokens=0) -> int:
    return int(lib().pkv_mla_decode_workspace_size(batch, num_heads, max_blocks_per_seq, block_size,
                                                   int(split_tokens)))


def mla_decode_plan(batch, num_heads, max_blocks_per_seq, block_size, split_tokens=0):
    a, b = ctypes.c_int32(), ctypes.c_int32()
    st = lib().pkv_mla_decode_plan(batch, num_heads, max_blocks_per_seq, block_size, int(split_tokens),
                                   ctypes.byref(a), ctypes.byref(b))
    _check(st, "pkv_mla_decode_plan")
    return {"split_tokens": a.value, "num_splits": b.value}


def mla_decode(q_latent, q_rope, cache: MLACache, block_table, context_lengths, scale, *, out=None,
               lse_out=None, workspace=None, split_tokens=0, stream=None):
    """Latent attention of one query per sequence: ``q_latent`` bf16 ``[B, H, 512]``, ``q_rope``
    bf16 ``[B, H, 64]``; returns bf16 ``[B, H, 512]``."""
    batch, heads = int(q_latent.shape[0]), int(q_latent.shape[1])
    mbs = int(block_table.shape[1])
    if out is None:
        out = torch.empty_like(q_latent)
    need = mla_decode_workspace_size(batch, heads, mbs, cache.block_size, split_tokens)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q_latent.device)  # no initial contents needed
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().pkv_mla_decode(_ptr(q_latent), _ptr(q_rope), heads, cache.ref, _ptr(block_table), mbs,
                              _ptr(context_lengths), batch, float(scale), _ptr(out), _ptr(lse_out),
                              _ptr(workspace), ws_bytes, int(split_tokens), _stream(stream))
    _check(st, "pkv_mla_decode")
    return out
