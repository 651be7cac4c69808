"""Python binding of libpkv (include/pkv.h): argument marshalling only.

Every step of the store / dequant / decode path runs in the HIP kernels of ``libpkv.so``; this
module passes device pointers (``tensor.data_ptr()``) and the current HIP stream, and raises
``PkvError`` on a non-zero status.  PyTorch supplies device memory and streams.

Before any call reaches the library, every tensor argument is checked on the host for dtype, shape,
contiguity and device (``ValueError`` otherwise): the kernels trust the sizes they are given, so a
wrong one would make them read or write out of bounds.  Outputs and scratch space that this module
allocates itself are allocated on the stream the call runs on, so the caching allocator cannot hand
their memory to other work while the kernels still use it.

There is no fallback: if ``libpkv.so`` has not been built, ``lib()`` raises.

Debug-only environment overrides (read at each call): ``PKV_CHECK=1`` runs ``check_indices`` (the
device-side bounds check of the block table, context lengths, query-length prefix sums and slot
mapping) before every store, dequant, walk and decode call and raises ``PkvIndexError`` instead of
making a call that would read out of bounds (it waits for the GPU: tests and debugging only);
``PKV_SPLIT_TOKENS=n`` and ``PKV_DECODE_PATH=valu|mfma|c8|tile`` stand in for the GQA decode's
``split_tokens`` and ``kernel`` arguments where a call leaves them at 0.
"""
from __future__ import annotations

import ctypes
import os

import torch  # loaded first: libpkv binds to the HIP runtime torch has already loaded

__all__ = ["PkvError", "PkvIndexError", "check_indices", "CHECK_CONTEXT", "CHECK_BLOCK", "CHECK_QLEN",
           "CHECK_SLOT", "Cache", "lib", "store_c8", "dequant", "decode_gqa", "decode_gqa_noalloc", "store_decode_gqa", "cache_walk",
           "decode_workspace_size", "NOALLOC_SCRATCH_BYTES",
           "decode_plan", "MLACache", "mla_store_c8", "mla_decode", "mla_store_decode", "mla_decode_workspace_size", "mla_cache_walk",
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
           "pkv_mla_decode_workspace_size", "pkv_mla_decode_plan", "pkv_mla_decode", "pkv_decode_gqa_noalloc",
           "pkv_store_decode_gqa", "pkv_cache_walk", "pkv_check_indices", "pkv_mla_store_decode",
           "pkv_mla_cache_walk")

NOALLOC_SCRATCH_BYTES = 32 << 20  # PKV_NOALLOC_SCRATCH_BYTES

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
        L.pkv_cache_walk.argtypes = [P, P, I32, P, I32, I32, I32, P, P]
        L.pkv_cache_walk.restype = ctypes.c_int
        L.pkv_check_indices.argtypes = [I32, I32, P, I32, P, P, I32, I32, P, I32, P, P]
        L.pkv_check_indices.restype = ctypes.c_int
        L.pkv_decode_workspace_size.argtypes = [I32, I32, I32, I32, I32, I32, I32, I32, P]
        L.pkv_decode_workspace_size.restype = SZ
        L.pkv_decode_gqa.argtypes = [P, I32, P, P, I32, P, P, I32, I32, ctypes.c_float, P, P, P, SZ,
                                     P, P]
        L.pkv_decode_gqa.restype = ctypes.c_int
        L.pkv_decode_gqa_noalloc.argtypes = [P, I32, P, P, I32, P, P, I32, I32, ctypes.c_float, P, P, P, P]
        L.pkv_decode_gqa_noalloc.restype = ctypes.c_int
        L.pkv_store_decode_gqa.argtypes = [P, P, P, I32, P, P, I32, P, I32, ctypes.c_float, P, P, P, SZ, P, P]
        L.pkv_store_decode_gqa.restype = ctypes.c_int
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
        L.pkv_mla_store_decode.argtypes = [P, P, P, P, I32, P, P, I32, P, I32, ctypes.c_float, P, P, P, SZ, I32, P]
        L.pkv_mla_store_decode.restype = ctypes.c_int
        L.pkv_mla_cache_walk.argtypes = [P, P, I32, P, I32, I32, P, P]
        L.pkv_mla_cache_walk.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _on_stream(stream):
    """Context in which this module allocates the tensors a call will use on ``stream``."""
    import contextlib

    return contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)


def _want(t, name, dtype, shape=None, ndim=None, optional=False):
    """Host-side check of one tensor argument: dtype, shape (None entries match any size),
    contiguity.  The device is checked separately (``_same_device``), after every shape, so that
    a wrong shape is reported as such whatever the device."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name}: {t.dim()} dimensions, expected {ndim}")
    if shape is not None:
        if t.dim() != len(shape) or any(w is not None and int(g) != int(w) for g, w in zip(t.shape, shape)):
            want = "[" + ", ".join("*" if w is None else str(int(w)) for w in shape) + "]"
            raise ValueError(f"{name}: shape {list(t.shape)}, expected {want}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _same_device(ref, **tensors):
    """Every given tensor on the GPU that holds ``ref`` (the cache)."""
    if ref.device.type != "cuda":
        raise ValueError(f"the cache is on {ref.device}: libpkv works on GPU memory only")
    for name, t in tensors.items():
        if t is not None and t.device != ref.device:
            raise ValueError(f"{name} is on {t.device}, the cache on {ref.device}")


def _check(status, what):
    if status != 0:
        raise PkvError(status, what)


PARTITION_PLANNED, PARTITION_FIXED, PARTITION_BALANCED = 0, 1, 2

CHECK_CONTEXT, CHECK_BLOCK, CHECK_QLEN, CHECK_SLOT = 1, 2, 4, 8  # PKV_CHECK_* of include/pkv.h


class PkvIndexError(ValueError):
    """An index array failed ``check_indices`` (raised under ``PKV_CHECK=1`` before the call)."""


def check_indices(cache, block_table=None, context_lengths=None, *, cu_q_lens=None, max_q_len=0,
                  slot_mapping=None, stream=None):
    """Bounds-check on the device the index arrays a call on ``cache`` (a ``Cache`` or ``MLACache``)
    would read; waits for the result.  Returns ``(flags, first_sequence, first_token)``: the
    ``CHECK_*`` bits of every violated condition (0 when all hold) and the lowest offending
    sequence and slot-mapping token (-1: none)."""
    ref = cache.k if isinstance(cache, Cache) else cache.latent
    _want(context_lengths, "context_lengths", torch.int32, ndim=1, optional=True)
    batch = int(context_lengths.shape[0]) if context_lengths is not None else \
        (int(cu_q_lens.shape[0]) - 1 if cu_q_lens is not None else 0)
    _want(block_table, "block_table", torch.int32, (batch, None), optional=True)
    _want(cu_q_lens, "cu_q_lens", torch.int32, (batch + 1,), optional=True)
    _want(slot_mapping, "slot_mapping", torch.int64, ndim=1, optional=True)
    _same_device(ref, block_table=block_table, context_lengths=context_lengths, cu_q_lens=cu_q_lens,
                 slot_mapping=slot_mapping)
    with _on_stream(stream):
        result = torch.empty(4, dtype=torch.int32, device=ref.device)
    mbs = int(block_table.shape[1]) if block_table is not None else 0
    ntok = int(slot_mapping.shape[0]) if slot_mapping is not None else 0
    st = lib().pkv_check_indices(cache.num_blocks, cache.block_size, _ptr(block_table), mbs,
                                 _ptr(context_lengths), _ptr(cu_q_lens), int(max_q_len), batch,
                                 _ptr(slot_mapping), ntok, _ptr(result), _stream(stream))
    _check(st, "pkv_check_indices")
    r = result.cpu().tolist()  # (waits for the check)
    return int(r[0]), int(r[1]), int(r[2])


def _debug_check(cache, what, **arrays):
    """Under PKV_CHECK=1: raise PkvIndexError before ``what`` if its index arrays are out of range."""
    if os.environ.get("PKV_CHECK", "0") in ("", "0"):
        return
    flags, seq, tok = check_indices(cache, **arrays)
    if flags:
        names = [n for n, bit in (("context length", CHECK_CONTEXT), ("block-table entry", CHECK_BLOCK),
                                  ("query lengths", CHECK_QLEN), ("slot mapping", CHECK_SLOT)) if flags & bit]
        where = f"sequence {seq}" if seq >= 0 else f"token {tok}"
        raise PkvIndexError(f"{what}: {', '.join(names)} out of range (first at {where}; PKV_CHECK flags {flags})")


_DECODE_PATHS = {"valu": 1, "mfma": 2, "c8": 3, "tile": 4}


def _opts(split_tokens=0, kernel=0, partition=0, window=0):
    if int(split_tokens) == 0 and os.environ.get("PKV_SPLIT_TOKENS"):
        split_tokens = int(os.environ["PKV_SPLIT_TOKENS"])
    if int(kernel) == 0 and os.environ.get("PKV_DECODE_PATH"):
        path = os.environ["PKV_DECODE_PATH"]
        if path not in _DECODE_PATHS:
            raise ValueError(f"PKV_DECODE_PATH={path!r}: expected one of {sorted(_DECODE_PATHS)}")
        kernel = _DECODE_PATHS[path]
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
        _want(self.k, "cache.k", dt, shape_k)
        _want(self.v, "cache.v", dt, shape_v)
        if sshape is not None:
            _want(self.k_scale, "cache.k_scale", torch.float32, sshape)
            _want(self.v_scale, "cache.v_scale", torch.float32, sshape)
        for t in (self.v, self.k_scale, self.v_scale):
            if t is not None and t.device != self.k.device:
                raise ValueError("cache tensors must share one device")
        self._c = _CacheT(self.k.data_ptr(), self.v.data_ptr(), _ptr(self.k_scale), _ptr(self.v_scale),
                          self.num_blocks, self.num_kv_heads, self.block_size, self.head_dim,
                          self.quant_mode)

    @property
    def ref(self):
        return ctypes.byref(self._c)


def store_c8(cache: Cache, k_new, v_new, *, slot_mapping=None, cu_q_lens=None, context_lengths=None,
             block_table=None, max_q_len=0, stream=None):
    """Quantize (or copy, mode 2) bf16 ``[T, Hkv, D]`` tokens into the cache."""
    _want(k_new, "k_new", torch.bfloat16, (None, cache.num_kv_heads, cache.head_dim))
    t = int(k_new.shape[0])
    _want(v_new, "v_new", torch.bfloat16, (t, cache.num_kv_heads, cache.head_dim))
    if slot_mapping is not None:
        _want(slot_mapping, "slot_mapping", torch.int64, (t,))
        batch, mbs = 0, 0
        for name, x in (("cu_q_lens", cu_q_lens), ("context_lengths", context_lengths), ("block_table", block_table)):
            if x is not None:
                raise ValueError(f"{name} must be None when slot_mapping is given")
    else:
        _want(context_lengths, "context_lengths", torch.int32, ndim=1)
        batch = int(context_lengths.shape[0])
        _want(block_table, "block_table", torch.int32, (batch, None))
        mbs = int(block_table.shape[1])
        _want(cu_q_lens, "cu_q_lens", torch.int32, (batch + 1,), optional=True)
        if cu_q_lens is None and t != batch:
            raise ValueError(f"without cu_q_lens every sequence stores one token: {t} tokens for {batch} sequences")
    _same_device(cache.k, k_new=k_new, v_new=v_new, slot_mapping=slot_mapping, cu_q_lens=cu_q_lens,
                 context_lengths=context_lengths, block_table=block_table)
    _debug_check(cache, "pkv_store_c8", block_table=block_table, context_lengths=context_lengths,
                 cu_q_lens=cu_q_lens, max_q_len=max_q_len, slot_mapping=slot_mapping)
    st = lib().pkv_store_c8(cache.ref, _ptr(k_new), _ptr(v_new), t, _ptr(slot_mapping), _ptr(cu_q_lens),
                            _ptr(context_lengths), _ptr(block_table), batch, mbs, int(max_q_len),
                            cache.quant_mode, _stream(stream))
    _check(st, "pkv_store_c8")


def dequant(cache: Cache, block_table, context_lengths, *, seq_offsets=None, k_out=None, v_out=None,
            token_stride=None, head_stride=None, num_rows=None, stream=None):
    """Gather to bf16 rows.  Default outputs: packed ``[num_rows, Hkv, D]`` tensors; without
    ``num_rows`` (the rows the sequences span) the lengths are read back to size them, which waits
    for the GPU.  Given outputs must hold every row the lengths and offsets address (a precondition,
    like the lengths themselves: the library does not read them on the host)."""
    _want(context_lengths, "context_lengths", torch.int32, ndim=1)
    batch = int(context_lengths.shape[0])
    _want(block_table, "block_table", torch.int32, (batch, None))
    _want(seq_offsets, "seq_offsets", torch.int64, (batch,), optional=True)
    _want(k_out, "k_out", torch.bfloat16, optional=True)
    _want(v_out, "v_out", torch.bfloat16, optional=True)
    _same_device(cache.k, block_table=block_table, context_lengths=context_lengths, seq_offsets=seq_offsets,
                 k_out=k_out, v_out=v_out)
    _debug_check(cache, "pkv_dequant", block_table=block_table, context_lengths=context_lengths)
    if k_out is None and v_out is None:
        if num_rows is None:  # (sizing from the lengths synchronises with the GPU)
            num_rows = int(context_lengths.sum().item()) if seq_offsets is None else \
                int((seq_offsets + context_lengths.to(seq_offsets.dtype)).max().item())
        with _on_stream(stream):
            k_out = torch.empty((max(int(num_rows), 1), cache.num_kv_heads, cache.head_dim), dtype=torch.bfloat16,
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


def cache_walk(cache: Cache, block_table, context_lengths, split_tokens, *, depth=1, out=None, stream=None):
    """Read what the int8 decode of these sequences reads from the cache, with ``split_tokens`` keys
    per wave, and nothing more (a read-ceiling measurement).  Returns the per-wave word sums, uint32
    bit patterns in an int32 tensor ``[batch, Hkv, nsplit]``."""
    _want(context_lengths, "context_lengths", torch.int32, ndim=1)
    batch = int(context_lengths.shape[0])
    _want(block_table, "block_table", torch.int32, (batch, None))
    mbs = int(block_table.shape[1])
    nsplit = -(-mbs * cache.block_size // int(split_tokens)) if split_tokens > 0 else 0
    _want(out, "out", torch.int32, (batch, cache.num_kv_heads, nsplit), optional=True)
    _same_device(cache.k, block_table=block_table, context_lengths=context_lengths, out=out)
    if out is None:
        with _on_stream(stream):
            out = torch.empty((batch, cache.num_kv_heads, max(nsplit, 1)), dtype=torch.int32, device=cache.k.device)
    _debug_check(cache, "pkv_cache_walk", block_table=block_table, context_lengths=context_lengths)
    st = lib().pkv_cache_walk(cache.ref, _ptr(block_table), mbs, _ptr(context_lengths), batch, int(split_tokens),
                              int(depth), _ptr(out), _stream(stream))
    _check(st, "pkv_cache_walk")
    return out


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
    _want(q, "q", torch.bfloat16, (None, None, cache.head_dim))
    tq, hq = int(q.shape[0]), int(q.shape[1])
    if hq % cache.num_kv_heads != 0:
        raise ValueError(f"{hq} query heads are not a multiple of {cache.num_kv_heads} KV heads")
    _want(context_lengths, "context_lengths", torch.int32, ndim=1)
    batch = int(context_lengths.shape[0])
    _want(block_table, "block_table", torch.int32, (batch, None))
    mbs = int(block_table.shape[1])
    _want(cu_q_lens, "cu_q_lens", torch.int32, (batch + 1,), optional=True)
    if cu_q_lens is None:
        max_q_len = 1
        if tq != batch:
            raise ValueError(f"without cu_q_lens q holds one row per sequence: {tq} rows for {batch} sequences")
    _want(out, "out", torch.bfloat16, (tq, hq, cache.head_dim), optional=True)
    _want(lse_out, "lse_out", torch.float32, (tq, hq), optional=True)
    _want(workspace, "workspace", torch.uint8, ndim=1, optional=True)
    _same_device(cache.k, q=q, block_table=block_table, context_lengths=context_lengths, cu_q_lens=cu_q_lens,
                 out=out, lse_out=lse_out, workspace=workspace)
    o = _opts(split_tokens, kernel, partition, window)
    need = int(lib().pkv_decode_workspace_size(batch, hq, cache.num_kv_heads, cache.head_dim, mbs,
                                               cache.block_size, max_q_len, cache.quant_mode,
                                               ctypes.byref(o)))
    with _on_stream(stream):
        if out is None:
            out = torch.empty_like(q)
        if workspace is None and need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)  # no initial contents needed
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _debug_check(cache, "pkv_decode_gqa", block_table=block_table, context_lengths=context_lengths,
                 cu_q_lens=cu_q_lens, max_q_len=max_q_len)
    st = lib().pkv_decode_gqa(_ptr(q), hq, cache.ref, _ptr(block_table), mbs, _ptr(context_lengths),
                              _ptr(cu_q_lens), batch, int(max_q_len), float(scale), _ptr(out),
                              _ptr(lse_out), _ptr(workspace), ws_bytes, ctypes.byref(o), _stream(stream))
    _check(st, "pkv_decode_gqa")
    return out


def store_decode_gqa(q, k_new, v_new, cache: Cache, block_table, context_lengths, scale, *, out=None,
                     lse_out=None, workspace=None, split_tokens=0, kernel=0, partition=0, window=0, stream=None):
    """One decode step: store each sequence's new token (bf16 ``[B, Hkv, D]``, at position
    ``context_lengths[b] - 1``) and attend with its one query ``q`` (bf16 ``[B, Hq, D]``)."""
    _want(q, "q", torch.bfloat16, (None, None, cache.head_dim))
    batch, hq = int(q.shape[0]), int(q.shape[1])
    if hq % cache.num_kv_heads != 0:
        raise ValueError(f"{hq} query heads are not a multiple of {cache.num_kv_heads} KV heads")
    _want(k_new, "k_new", torch.bfloat16, (batch, cache.num_kv_heads, cache.head_dim))
    _want(v_new, "v_new", torch.bfloat16, (batch, cache.num_kv_heads, cache.head_dim))
    _want(context_lengths, "context_lengths", torch.int32, (batch,))
    _want(block_table, "block_table", torch.int32, (batch, None))
    mbs = int(block_table.shape[1])
    _want(out, "out", torch.bfloat16, (batch, hq, cache.head_dim), optional=True)
    _want(lse_out, "lse_out", torch.float32, (batch, hq), optional=True)
    _want(workspace, "workspace", torch.uint8, ndim=1, optional=True)
    _same_device(cache.k, q=q, k_new=k_new, v_new=v_new, block_table=block_table, context_lengths=context_lengths,
                 out=out, lse_out=lse_out, workspace=workspace)
    o = _opts(split_tokens, kernel, partition, window)
    need = int(lib().pkv_decode_workspace_size(batch, hq, cache.num_kv_heads, cache.head_dim, mbs,
                                               cache.block_size, 1, cache.quant_mode, ctypes.byref(o)))
    with _on_stream(stream):
        if out is None:
            out = torch.empty_like(q)
        if workspace is None and need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)  # no initial contents needed
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _debug_check(cache, "pkv_store_decode_gqa", block_table=block_table, context_lengths=context_lengths)
    st = lib().pkv_store_decode_gqa(_ptr(q), _ptr(k_new), _ptr(v_new), hq, cache.ref, _ptr(block_table), mbs,
                                    _ptr(context_lengths), batch, float(scale), _ptr(out), _ptr(lse_out),
                                    _ptr(workspace), ws_bytes, ctypes.byref(o), _stream(stream))
    _check(st, "pkv_store_decode_gqa")
    return out


def decode_gqa_noalloc(q, cache: Cache, block_table, context_lengths, scale, out, *, cu_q_lens=None, max_q_len=1,
                       lse_out=None, split_tokens=0, kernel=0, partition=0, window=0, stream=None):
    """``decode_gqa`` through ``pkv_decode_gqa_noalloc``: no workspace, and nothing allocated here
    either (``out`` is required).  Its scratch space is one fixed array per GPU, shared by every
    such call on that GPU (calls that overlap in time race)."""
    _want(q, "q", torch.bfloat16, (None, None, cache.head_dim))
    tq, hq = int(q.shape[0]), int(q.shape[1])
    if hq % cache.num_kv_heads != 0:
        raise ValueError(f"{hq} query heads are not a multiple of {cache.num_kv_heads} KV heads")
    _want(context_lengths, "context_lengths", torch.int32, ndim=1)
    batch = int(context_lengths.shape[0])
    _want(block_table, "block_table", torch.int32, (batch, None))
    _want(cu_q_lens, "cu_q_lens", torch.int32, (batch + 1,), optional=True)
    if cu_q_lens is None:
        max_q_len = 1
        if tq != batch:
            raise ValueError(f"without cu_q_lens q holds one row per sequence: {tq} rows for {batch} sequences")
    _want(out, "out", torch.bfloat16, (tq, hq, cache.head_dim))
    _want(lse_out, "lse_out", torch.float32, (tq, hq), optional=True)
    _same_device(cache.k, q=q, block_table=block_table, context_lengths=context_lengths, cu_q_lens=cu_q_lens,
                 out=out, lse_out=lse_out)
    o = _opts(split_tokens, kernel, partition, window)
    _debug_check(cache, "pkv_decode_gqa_noalloc", block_table=block_table, context_lengths=context_lengths,
                 cu_q_lens=cu_q_lens, max_q_len=max_q_len)
    st = lib().pkv_decode_gqa_noalloc(_ptr(q), hq, cache.ref, _ptr(block_table), int(block_table.shape[1]),
                                      _ptr(context_lengths), _ptr(cu_q_lens), batch, int(max_q_len), float(scale),
                                      _ptr(out), _ptr(lse_out), ctypes.byref(o), _stream(stream))
    _check(st, "pkv_decode_gqa_noalloc")
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
    _want(latent_new, "latent_new", torch.bfloat16, (None, cache.latent_dim))
    t = int(latent_new.shape[0])
    _want(rope_new, "rope_new", torch.bfloat16, (t, cache.rope_dim))
    if slot_mapping is not None:
        _want(slot_mapping, "slot_mapping", torch.int64, (t,))
        batch, mbs = 0, 0
    else:
        _want(context_lengths, "context_lengths", torch.int32, ndim=1)
        batch = int(context_lengths.shape[0])
        _want(block_table, "block_table", torch.int32, (batch, None))
        mbs = int(block_table.shape[1])
        _want(cu_q_lens, "cu_q_lens", torch.int32, (batch + 1,), optional=True)
        if cu_q_lens is None and t != batch:
            raise ValueError(f"without cu_q_lens every sequence stores one token: {t} tokens for {batch} sequences")
    _same_device(cache.latent, latent_new=latent_new, rope_new=rope_new, slot_mapping=slot_mapping,
                 cu_q_lens=cu_q_lens, context_lengths=context_lengths, block_table=block_table)
    _debug_check(cache, "pkv_mla_store_c8", block_table=block_table, context_lengths=context_lengths,
                 cu_q_lens=cu_q_lens, slot_mapping=slot_mapping)
    st = lib().pkv_mla_store_c8(cache.ref, _ptr(latent_new), _ptr(rope_new), t, _ptr(slot_mapping),
                                _ptr(cu_q_lens), _ptr(context_lengths), _ptr(block_table), batch, mbs,
                                _stream(stream))
    _check(st, "pkv_mla_store_c8")


def mla_cache_walk(cache: MLACache, block_table, context_lengths, split_tokens, *, out=None, stream=None):
    """Read what the MLA decode of these sequences reads from the latent cache, ``split_tokens`` keys
    per workgroup, and nothing more (a read-ceiling measurement).  Returns the per-workgroup word
    sums, uint32 bit patterns in an int32 tensor ``[batch, nsplit]``."""
    _want(context_lengths, "context_lengths", torch.int32, ndim=1)
    batch = int(context_lengths.shape[0])
    _want(block_table, "block_table", torch.int32, (batch, None))
    mbs = int(block_table.shape[1])
    nsplit = -(-mbs * cache.block_size // int(split_tokens)) if split_tokens > 0 else 0
    _want(out, "out", torch.int32, (batch, nsplit), optional=True)
    _same_device(cache.latent, block_table=block_table, context_lengths=context_lengths, out=out)
    if out is None:
        with _on_stream(stream):
            out = torch.empty((batch, max(nsplit, 1)), dtype=torch.int32, device=cache.latent.device)
    _debug_check(cache, "pkv_mla_cache_walk", block_table=block_table, context_lengths=context_lengths)
    st = lib().pkv_mla_cache_walk(cache.ref, _ptr(block_table), mbs, _ptr(context_lengths), batch,
                                  int(split_tokens), _ptr(out), _stream(stream))
    _check(st, "pkv_mla_cache_walk")
    return out


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
    _want(q_latent, "q_latent", torch.bfloat16, (None, None, cache.latent_dim))
    batch, heads = int(q_latent.shape[0]), int(q_latent.shape[1])
    _want(q_rope, "q_rope", torch.bfloat16, (batch, heads, cache.rope_dim))
    _want(context_lengths, "context_lengths", torch.int32, (batch,))
    _want(block_table, "block_table", torch.int32, (batch, None))
    mbs = int(block_table.shape[1])
    _want(out, "out", torch.bfloat16, (batch, heads, cache.latent_dim), optional=True)
    _want(lse_out, "lse_out", torch.float32, (batch, heads), optional=True)
    _want(workspace, "workspace", torch.uint8, ndim=1, optional=True)
    _same_device(cache.latent, q_latent=q_latent, q_rope=q_rope, context_lengths=context_lengths,
                 block_table=block_table, out=out, lse_out=lse_out, workspace=workspace)
    need = mla_decode_workspace_size(batch, heads, mbs, cache.block_size, split_tokens)
    with _on_stream(stream):
        if out is None:
            out = torch.empty_like(q_latent)
        if workspace is None and need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=q_latent.device)  # no initial contents needed
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _debug_check(cache, "pkv_mla_decode", block_table=block_table, context_lengths=context_lengths)
    st = lib().pkv_mla_decode(_ptr(q_latent), _ptr(q_rope), heads, cache.ref, _ptr(block_table), mbs,
                              _ptr(context_lengths), batch, float(scale), _ptr(out), _ptr(lse_out),
                              _ptr(workspace), ws_bytes, int(split_tokens), _stream(stream))
    _check(st, "pkv_mla_decode")
    return out


def mla_store_decode(q_latent, q_rope, latent_new, rope_new, cache: MLACache, block_table, context_lengths, scale,
                     *, out=None, lse_out=None, workspace=None, split_tokens=0, stream=None):
    """One MLA decode step: store each sequence's new latent row (bf16 ``[B, 512]``) and rotary row
    (bf16 ``[B, 64]``) at position ``context_lengths[b] - 1``, then attend with its query."""
    _want(q_latent, "q_latent", torch.bfloat16, (None, None, cache.latent_dim))
    batch, heads = int(q_latent.shape[0]), int(q_latent.shape[1])
    _want(q_rope, "q_rope", torch.bfloat16, (batch, heads, cache.rope_dim))
    _want(latent_new, "latent_new", torch.bfloat16, (batch, cache.latent_dim))
    _want(rope_new, "rope_new", torch.bfloat16, (batch, cache.rope_dim))
    _want(context_lengths, "context_lengths", torch.int32, (batch,))
    _want(block_table, "block_table", torch.int32, (batch, None))
    mbs = int(block_table.shape[1])
    _want(out, "out", torch.bfloat16, (batch, heads, cache.latent_dim), optional=True)
    _want(lse_out, "lse_out", torch.float32, (batch, heads), optional=True)
    _want(workspace, "workspace", torch.uint8, ndim=1, optional=True)
    _same_device(cache.latent, q_latent=q_latent, q_rope=q_rope, latent_new=latent_new, rope_new=rope_new,
                 context_lengths=context_lengths, block_table=block_table, out=out, lse_out=lse_out,
                 workspace=workspace)
    need = mla_decode_workspace_size(batch, heads, mbs, cache.block_size, split_tokens)
    with _on_stream(stream):
        if out is None:
            out = torch.empty_like(q_latent)
        if workspace is None and need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=q_latent.device)  # no initial contents needed
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _debug_check(cache, "pkv_mla_store_decode", block_table=block_table, context_lengths=context_lengths)
    st = lib().pkv_mla_store_decode(_ptr(q_latent), _ptr(q_rope), _ptr(latent_new), _ptr(rope_new), heads, cache.ref,
                                    _ptr(block_table), mbs, _ptr(context_lengths), batch, float(scale), _ptr(out),
                                    _ptr(lse_out), _ptr(workspace), ws_bytes, int(split_tokens), _stream(stream))
    _check(st, "pkv_mla_store_decode")
    return out
