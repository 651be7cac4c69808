"""Seeded synthetic inputs for the paged int8 KV-cache path.

This module only draws random numbers and lays out shapes: sequence lengths,
block tables, bf16 Q/K/V tensors and (for the per-channel cache mode) static
per-channel scales, which that mode takes as inputs.  It holds none of the method's arithmetic
(no quantization, no attention), so both the HIP path and the CPU oracle may
take their inputs from it.

Every workload is reproducible from one integer seed.  Sub-streams are derived
from it so that, e.g., changing the Q draw never changes the block table:

    stream 0  context / query lengths
    stream 1  block-table permutation
    stream 2  Q        stream 3  K        stream 4  V
    stream 5  outlier K channels
    stream 6  per-channel K scales    stream 7  per-channel V scales
    MLA workloads: stream 2 latent query, 8 rotary query, 3 latent rows, 9 rotary key rows

Integer draws use numpy's PCG64 (``numpy.random.default_rng``); the bf16
tensors use torch's seeded generator on the requested device followed by a
round-to-nearest-even cast to bfloat16.  Tensors drawn on different devices
differ, so a test draws once and copies what it needs.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

QUANT_PER_TOKEN = 0
QUANT_PER_BLOCK = 1
QUANT_NONE_BF16 = 2
QUANT_PER_CHANNEL = 3


def _rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(stream)])


def _torch_seed(seed: int, stream: int) -> int:
    return (int(seed) * 1_000_003 + int(stream) * 7919) & 0x7FFF_FFFF_FFFF


@dataclasses.dataclass
class Workload:
    """Shapes, lengths and block table of one synthetic batch.

    ``context_lengths[b]`` is the KV length of sequence b *after* the batch's
    new tokens are stored; the new tokens occupy positions
    ``[context_lengths[b] - q_lens[b], context_lengths[b])``.
    """

    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    quant_mode: int
    context_lengths: np.ndarray  # int32 [B]
    q_lens: np.ndarray  # int32 [B]
    num_blocks: int
    max_blocks_per_seq: int
    block_table: np.ndarray  # int32 [B, MBS], unused entries -1
    seed: int
    k_outlier_channels: Optional[np.ndarray] = None  # int64 [n, 2] of (kvh, d)
    k_outlier_factor: float = 8.0
    decode_only: bool = True  # q_len == 1 for every sequence, no cu_q_lens

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def prior_lengths(self) -> np.ndarray:
        return (self.context_lengths - self.q_lens).astype(np.int32)

    @property
    def num_new_tokens(self) -> int:
        return int(self.q_lens.sum())

    @property
    def total_tokens(self) -> int:
        return int(self.context_lengths.sum())

    @property
    def max_q_len(self) -> int:
        return int(self.q_lens.max()) if self.batch else 0

    @property
    def cu_q_lens(self) -> np.ndarray:
        cu = np.zeros(self.batch + 1, dtype=np.int32)
        cu[1:] = np.cumsum(self.q_lens)
        return cu

    @property
    def cu_prior(self) -> np.ndarray:
        cu = np.zeros(self.batch + 1, dtype=np.int64)
        cu[1:] = np.cumsum(self.prior_lengths)
        return cu

    @property
    def cu_context(self) -> np.ndarray:
        cu = np.zeros(self.batch + 1, dtype=np.int64)
        cu[1:] = np.cumsum(self.context_lengths)
        return cu


def make_block_table(context_lengths, block_size, num_blocks, max_blocks_per_seq, seed):
    """Sequence b takes consecutive entries of a seeded permutation of the pool."""
    perm = _rng(seed, 1).permutation(num_blocks).astype(np.int32)
    bt = np.full((len(context_lengths), max_blocks_per_seq), -1, dtype=np.int32)
    pos = 0
    for b, c in enumerate(context_lengths):
        nb = -(-int(c) // block_size)
        if nb > max_blocks_per_seq or pos + nb > num_blocks:
            raise ValueError("pool too small for the requested lengths")
        bt[b, :nb] = perm[pos:pos + nb]
        pos += nb
    return bt


def custom_workload(name, *, batch, num_q_heads, num_kv_heads, head_dim, block_size,
                    quant_mode, context_lengths, q_lens=None, seed=0, pool_factor=2,
                    num_blocks=None, max_blocks_per_seq=None, outlier_fraction=0.0,
                    decode_only=None):
    ctx = np.asarray(context_lengths, dtype=np.int32).reshape(batch)
    ql = np.minimum(ctx, 1).astype(np.int32) if q_lens is None else np.asarray(q_lens, np.int32).reshape(batch)
    if np.any(ql > ctx):
        raise ValueError("q_len exceeds context length")
    need = int(sum(-(-int(c) // block_size) for c in ctx))
    if num_blocks is None:
        num_blocks = max(1, pool_factor * need)
    if max_blocks_per_seq is None:
        max_blocks_per_seq = max(1, max(-(-int(c) // block_size) for c in ctx) if batch else 1)
    bt = make_block_table(ctx, block_size, num_blocks, max_blocks_per_seq, seed)
    outl = None
    if outlier_fraction > 0:
        n = int(round(outlier_fraction * num_kv_heads * head_dim))
        flat = _rng(seed, 5).choice(num_kv_heads * head_dim, size=n, replace=False)
        outl = np.stack([flat // head_dim, flat % head_dim], axis=1).astype(np.int64)
    if decode_only is None:
        decode_only = bool(np.all(ql == np.minimum(ctx, 1)))
    return Workload(name, batch, num_q_heads, num_kv_heads, head_dim, block_size, quant_mode,
                    ctx, ql, int(num_blocks), int(max_blocks_per_seq), bt, seed, outl,
                    decode_only=decode_only)


CONFIG_NAMES = [
    "tiny-decode",
    "qwen3-8b-decode",
    "long-context-decode",
    "bf16-large-batch-decode",
    "chunked-store-multitoken",
    "paged-prefill",
]


def make_config(index: int, seed: Optional[int] = None, quant_mode: Optional[int] = None,
                prompt_len: int = 0) -> Workload:
    """The five benchmark workloads, seeded with ``1000 + index`` by default.

    0  tiny:        B=2, 8/2 heads, D=64, BS=16, ctx {37, 100}, pool = permutation of 16 blocks
    1  Qwen3-8B:    B=32, 32/8 heads, D=128, BS=16, ctx ~ U[1024, 4096], 1% of K channels x8
    2  long ctx:    B=8, 64/8 heads, D=128, BS=128, ctx ~ U[32768, 131072]
    3  bf16 cache:  B=256, 32/8 heads, D=128, BS=16, ctx log-normal (median 1024, sigma 1),
                    clipped to [64, 8192]
    4  chunked:     B=64, q_len ~ U[1, 16], prior ~ U[0, 16384], 40/8 heads, D=128, BS=16,
                    one fp32 scale per 16-token block
    5  prefill:     B=4 prompts of 2048 tokens (store and causal attention of every token),
                    32/8 heads, D=128, BS=16, per-token scales (a measurement workload for the
                    paged-prefill row, not one of the five above); prompt_len > 0: prompts of
                    that many tokens instead, max(1, 8192 // prompt_len) of them
    """
    if quant_mode is not None:  # the same shapes and lengths with another cache mode
        w = make_config(index, seed, prompt_len=prompt_len)
        return dataclasses.replace(w, quant_mode=int(quant_mode), name=f"{w.name}-mode{int(quant_mode)}")
    s = 1000 + index if seed is None else seed
    r = _rng(s, 0)
    if index == 0:
        return custom_workload(CONFIG_NAMES[0], batch=2, num_q_heads=8, num_kv_heads=2, head_dim=64,
                               block_size=16, quant_mode=QUANT_PER_TOKEN, context_lengths=[37, 100],
                               seed=s, num_blocks=16, max_blocks_per_seq=7)
    if index == 1:
        ctx = r.integers(1024, 4096, size=32, endpoint=True)
        return custom_workload(CONFIG_NAMES[1], batch=32, num_q_heads=32, num_kv_heads=8, head_dim=128,
                               block_size=16, quant_mode=QUANT_PER_TOKEN, context_lengths=ctx, seed=s,
                               max_blocks_per_seq=4096 // 16, outlier_fraction=0.01)
    if index == 2:
        ctx = r.integers(32768, 131072, size=8, endpoint=True)
        return custom_workload(CONFIG_NAMES[2], batch=8, num_q_heads=64, num_kv_heads=8, head_dim=128,
                               block_size=128, quant_mode=QUANT_PER_TOKEN, context_lengths=ctx, seed=s,
                               max_blocks_per_seq=131072 // 128)
    if index == 3:
        z = r.standard_normal(256)
        ctx = np.clip(np.round(np.exp(math.log(1024.0) + 1.0 * z)), 64, 8192).astype(np.int64)
        return custom_workload(CONFIG_NAMES[3], batch=256, num_q_heads=32, num_kv_heads=8, head_dim=128,
                               block_size=16, quant_mode=QUANT_NONE_BF16, context_lengths=ctx, seed=s,
                               max_blocks_per_seq=8192 // 16)
    if index == 4:
        ql = r.integers(1, 16, size=64, endpoint=True)
        prior = r.integers(0, 16384, size=64, endpoint=True)
        return custom_workload(CONFIG_NAMES[4], batch=64, num_q_heads=40, num_kv_heads=8, head_dim=128,
                               block_size=16, quant_mode=QUANT_PER_BLOCK, context_lengths=prior + ql,
                               q_lens=ql, seed=s, max_blocks_per_seq=-(-(16384 + 16) // 16),
                               decode_only=False)
    if index == 5:
        n = int(prompt_len) if prompt_len > 0 else 2048
        ctx = np.full(max(1, 8192 // n) if prompt_len > 0 else 4, n)
        name = CONFIG_NAMES[5] if prompt_len <= 0 else f"{CONFIG_NAMES[5]}-{n}"
        return custom_workload(name, batch=len(ctx), num_q_heads=32, num_kv_heads=8, head_dim=128,
                               block_size=16, quant_mode=QUANT_PER_TOKEN, context_lengths=ctx, q_lens=ctx,
                               seed=s, max_blocks_per_seq=-(-n // 16), decode_only=False)
    raise ValueError(f"no config {index}")


# ----------------------------------------------------------------------------------------------
# bf16 tensors
# ----------------------------------------------------------------------------------------------

def normal_bf16(shape, seed: int, stream: int, device="cpu"):
    """N(0, 1) drawn in fp32 by torch's seeded generator, cast to bf16 (round to nearest even)."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(_torch_seed(seed, stream))
    x = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    return x.to(torch.bfloat16)


def gen_tensors(w: Workload, device="cpu"):
    """Draw Q for the new tokens and K/V for every position of every sequence.

    Returns a dict of torch bf16 tensors:
      q      [Tq, Hq, D]      Tq = sum(q_lens) (= B for pure decode)
      k_all  [sum(ctx), Hkv, D]   sequence b's positions start at ``w.cu_context[b]``
      v_all  [sum(ctx), Hkv, D]
    The outlier channels of K (if any) are multiplied by ``w.k_outlier_factor``, a power of
    two, so the scaled values are exact in bf16.
    """
    import torch

    tq = w.num_new_tokens
    q = normal_bf16((tq, w.num_q_heads, w.head_dim), w.seed, 2, device)
    k = normal_bf16((w.total_tokens, w.num_kv_heads, w.head_dim), w.seed, 3, device)
    v = normal_bf16((w.total_tokens, w.num_kv_heads, w.head_dim), w.seed, 4, device)
    if w.k_outlier_channels is not None and len(w.k_outlier_channels):
        kv_idx = torch.as_tensor(w.k_outlier_channels[:, 0], device=device)
        d_idx = torch.as_tensor(w.k_outlier_channels[:, 1], device=device)
        k[:, kv_idx, d_idx] = k[:, kv_idx, d_idx] * w.k_outlier_factor
    out = {"q": q, "k_all": k, "v_all": v}
    if w.quant_mode == QUANT_PER_CHANNEL:
        out["k_scale"], out["v_scale"] = channel_scales(w, device)
    return out


def channel_scales(w: Workload, device="cpu"):
    """Static per-channel scales [Hkv, D] (fp32) for the per-channel cache mode, as a calibration
    would supply them: a seeded range of 3 to 4.5 standard deviations per channel over 127
    (N(0, 1) data; values beyond the range saturate), times the outlier factor on K's outlier
    channels."""
    import torch

    shape = (w.num_kv_heads, w.head_dim)
    ks = _rng(w.seed, 6).uniform(3.0, 4.5, size=shape).astype(np.float32) / np.float32(127)
    vs = _rng(w.seed, 7).uniform(3.0, 4.5, size=shape).astype(np.float32) / np.float32(127)
    if w.k_outlier_channels is not None and len(w.k_outlier_channels):
        ks[w.k_outlier_channels[:, 0], w.k_outlier_channels[:, 1]] *= np.float32(w.k_outlier_factor)
    return torch.from_numpy(ks).to(device), torch.from_numpy(vs).to(device)


def split_prior_new(w: Workload, t_all):
    """Index tensors selecting the prior tokens and the new tokens from a ``*_all`` tensor."""
    import torch

    prior_idx, new_idx = [], []
    cu = w.cu_context
    for b in range(w.batch):
        c, ql = int(w.context_lengths[b]), int(w.q_lens[b])
        prior_idx.append(np.arange(cu[b], cu[b] + c - ql))
        new_idx.append(np.arange(cu[b] + c - ql, cu[b] + c))
    pi = torch.as_tensor(np.concatenate(prior_idx) if prior_idx else np.zeros(0, np.int64),
                         device=t_all.device)
    ni = torch.as_tensor(np.concatenate(new_idx) if new_idx else np.zeros(0, np.int64),
                         device=t_all.device)
    return t_all.index_select(0, pi), t_all.index_select(0, ni)


def prior_workload_view(w: Workload):
    """Lengths for storing the prior tokens in one prefill-style call: q_len = prior, ctx = prior."""
    prior = w.prior_lengths
    return prior.copy(), prior.copy()


# ----------------------------------------------------------------------------------------------
# paged MLA (latent cache) workloads
# ----------------------------------------------------------------------------------------------

@dataclasses.dataclass
class MLAWorkload:
    """One decode batch over a paged latent cache: one new token (and query) per sequence, stored
    at position ``context_lengths[b] - 1``; every query head shares the sequence's latent rows."""

    name: str
    batch: int
    num_heads: int
    latent_dim: int
    rope_dim: int
    block_size: int
    context_lengths: np.ndarray  # int32 [B]
    num_blocks: int
    max_blocks_per_seq: int
    block_table: np.ndarray  # int32 [B, MBS], unused entries -1
    seed: int
    softmax_scale: float

    @property
    def total_tokens(self) -> int:
        return int(self.context_lengths.sum())

    @property
    def prior_lengths(self) -> np.ndarray:
        return np.maximum(self.context_lengths - 1, 0).astype(np.int32)

    @property
    def cu_context(self) -> np.ndarray:
        cu = np.zeros(self.batch + 1, dtype=np.int64)
        cu[1:] = np.cumsum(self.context_lengths)
        return cu


def mla_workload(name, *, batch, num_heads, block_size, context_lengths, latent_dim=512, rope_dim=64,
                 seed=0, pool_factor=2, num_blocks=None, max_blocks_per_seq=None, softmax_scale=None):
    ctx = np.asarray(context_lengths, dtype=np.int32).reshape(batch)
    need = int(sum(-(-int(c) // block_size) for c in ctx))
    if num_blocks is None:
        num_blocks = max(1, pool_factor * need)
    if max_blocks_per_seq is None:
        max_blocks_per_seq = max(1, max(-(-int(c) // block_size) for c in ctx) if batch else 1)
    bt = make_block_table(ctx, block_size, num_blocks, max_blocks_per_seq, seed)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(latent_dim + rope_dim)
    return MLAWorkload(name, batch, num_heads, latent_dim, rope_dim, block_size, ctx, int(num_blocks),
                       int(max_blocks_per_seq), bt, seed, float(softmax_scale))


MLA_CONFIG_NAMES = ["mla-tiny-decode", "deepseek-v3-mla-decode"]


def make_mla_config(index: int, seed: Optional[int] = None) -> MLAWorkload:
    """MLA decode workloads, seeded with ``2000 + index`` by default.

    0  tiny:       B=2, 16 heads, latent 512 + rotary 64, BS=16, ctx {37, 100}
    1  DeepSeek-V3 shaped: B=64, 16 query heads (one GPU's share when the 128 heads are split
                   8 ways; the latent cache is then read whole by every GPU), latent 512 +
                   rotary 64, BS=64, ctx ~ U[2048, 8192], softmax scale 1/sqrt(128 + 64) (the
                   per-head query-key width before absorption)
    """
    s = 2000 + index if seed is None else seed
    r = _rng(s, 0)
    if index == 0:
        return mla_workload(MLA_CONFIG_NAMES[0], batch=2, num_heads=16, block_size=16,
                            context_lengths=[37, 100], seed=s, num_blocks=16, max_blocks_per_seq=7)
    if index == 1:
        ctx = r.integers(2048, 8192, size=64, endpoint=True)
        return mla_workload(MLA_CONFIG_NAMES[1], batch=64, num_heads=16, block_size=64, context_lengths=ctx,
                            seed=s, max_blocks_per_seq=8192 // 64, softmax_scale=1.0 / math.sqrt(192.0))
    raise ValueError(f"no MLA config {index}")


def gen_mla_tensors(w: MLAWorkload, device="cpu"):
    """N(0, 1) bf16 draws: q_latent [B, H, Dc], q_rope [B, H, Dr], latent_all [sum(ctx), Dc],
    rope_all [sum(ctx), Dr] (sequence b's positions start at ``w.cu_context[b]``)."""
    return {
        "q_latent": normal_bf16((w.batch, w.num_heads, w.latent_dim), w.seed, 2, device),
        "q_rope": normal_bf16((w.batch, w.num_heads, w.rope_dim), w.seed, 8, device),
        "latent_all": normal_bf16((w.total_tokens, w.latent_dim), w.seed, 3, device),
        "rope_all": normal_bf16((w.total_tokens, w.rope_dim), w.seed, 9, device),
    }
