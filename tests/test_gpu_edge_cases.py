"""GPU parity on the method's degenerate and stressing inputs, against the CPU oracle.

* All-zero tokens (per-token and per-channel modes, the MLA store) and all-zero blocks (per-block
  mode, in the first chunk stored into a block and in a later one): the scale is 0 and every code
  0, with no epsilon (the reading of an absmax of 0); the decode over such keys and values.
* Softmax scale 0 (every visible key weighs the same: the output is the mean of the values) and
  negative scales, through every decode kernel and both key partitions.
* Query rows with one channel 64 and 256 times larger than the rest (outlier channels), which
  stress any kernel that rounds the query relative to its largest element.

Bars as in test_gpu_parity: codes and scales bit-exact; attention within 1e-2 (max-abs and
norm-relative); lse within 1e-4 + 1e-5 |lse| plus the fp32 evaluation bound (gpu_harness.lse_bar).
"""
import numpy as np
import pytest
import torch

import gen
import oracle
import paged_kv_cache_c8_amd as pkv
from tests.gpu_harness import Run, bits

pytestmark = pytest.mark.gpu

KERNELS = [1, 2, 3]


def _wl(mode, d, bs, g, ctx, ql=None, hkv=2, seed=0):
    return gen.custom_workload(f"edge-m{mode}-d{d}-bs{bs}-g{g}", batch=len(ctx), num_q_heads=hkv * g,
                               num_kv_heads=hkv, head_dim=d, block_size=bs, quant_mode=mode,
                               context_lengths=ctx, q_lens=ql, seed=seed)


def _kernels(mode):
    return [3] if mode == 3 else KERNELS


def _runs(mode, d, kws):
    """(kernel, options) pairs: every kernel serving the mode with each of the key-partition options,
    and the tile kernel (kernel 4: one pass over the keys, no partition options) where it serves
    (head_dim 128, per-token or per-block scales)."""
    runs = [(k, kw) for k in _kernels(mode) for kw in kws]
    if d == 128 and mode in (0, 1):
        runs.append((4, {}))
    return runs


def _zero_positions(w, t, which, seq_pos):
    """Zero the bf16 rows of ``which`` ("k", "v" or "kv") at (sequence, position, KV head) triples
    (head None: every head) in the drawn tensors, before anything is stored."""
    cu = w.cu_context
    for b, p, h in seq_pos:
        row = int(cu[b]) + p
        for name in (("k_all",) if which == "k" else ("v_all",) if which == "v" else ("k_all", "v_all")):
            if h is None:
                t[name][row].zero_()
            else:
                t[name][row, h].zero_()


@pytest.mark.parametrize("mode", [0, 3])
def test_all_zero_tokens_store_and_decode(mode):
    """Per-token (mode 0) and per-channel (mode 3) caches: tokens whose K row, V row or both are all
    zero, among the prior tokens and the decode step's new token; codes and scales bit-exact (scale
    0, codes 0), decode within the bar through every kernel that serves the mode."""
    ctx = [1, 17, 40, 300]
    w = _wl(mode, 128, 16, 4, ctx, seed=91 + mode)
    t = gen.gen_tensors(w, device=torch.device("cuda"))
    zeros_kv = [(0, 0, None), (1, 16, None), (2, 5, 0), (3, 299, None), (3, 100, 1)]  # 299: new token
    zeros_k = [(2, 39, 1), (3, 7, 0)]
    zeros_v = [(1, 3, None), (3, 8, 1)]
    _zero_positions(w, t, "kv", zeros_kv)
    _zero_positions(w, t, "k", zeros_k)
    _zero_positions(w, t, "v", zeros_v)
    r = Run(w, tensors=t)
    r.store_prior()
    r.store_new()
    r.assert_cache_equal()
    if mode == 0:  # the zero rows store scale 0 (on both sides: compared bit for bit above)
        ks = r.cache.k_scale.cpu().numpy()
        vs = r.cache.v_scale.cpu().numpy()
        for b, p, h in zeros_kv + zeros_k:
            blk, off = w.block_table[b, p // 16], p % 16
            assert np.all(ks[blk, slice(None) if h is None else h, off] == 0)
            assert np.all(r.cache.k[blk, slice(None) if h is None else h, off].cpu().numpy() == 0)
        for b, p, h in zeros_kv + zeros_v:
            blk, off = w.block_table[b, p // 16], p % 16
            assert np.all(vs[blk, slice(None) if h is None else h, off] == 0)
    ref = r.oracle_decode()
    for kernel, kw in _runs(mode, w.head_dim, (dict(), dict(split_tokens=128), dict(partition=2))):
        out, lse = r.decode(kernel=kernel, **kw)
        r.assert_decode_close(out, lse, ref)


def test_all_zero_blocks_per_block_mode():
    """Per-block scales (mode 1), a prior chunk then a new chunk of up to 16 tokens:
    sequence 0: block 1's prior tokens all zero (scale 0), then non-zero new tokens in it (the
    scale grows from 0; the old codes stay 0);
    sequence 1: non-zero prior, an all-zero new chunk (the scale stays, the new codes are 0; block 2
    is written only by zeros: scale 0);
    sequence 2: every value zero (every scale 0);
    sequence 3: ordinary values.  Codes and scales bit-exact, decode within the bar."""
    ctx, ql = [40, 40, 20, 70], [10, 10, 4, 16]
    w = _wl(1, 128, 16, 5, ctx, ql, seed=93)
    t = gen.gen_tensors(w, device=torch.device("cuda"))
    _zero_positions(w, t, "kv", [(0, p, None) for p in range(16, 30)])
    _zero_positions(w, t, "kv", [(1, p, None) for p in range(30, 40)])
    _zero_positions(w, t, "kv", [(2, p, None) for p in range(20)])
    r = Run(w, tensors=t)
    r.store_prior()
    torch.cuda.synchronize()
    ks_prior = r.cache.k_scale.cpu().numpy().copy()
    r.store_new()
    r.assert_cache_equal()
    ks = r.cache.k_scale.cpu().numpy()
    bt = w.block_table
    assert np.all(ks_prior[bt[0, 1]] == 0) and np.all(ks[bt[0, 1]] > 0)  # grew from 0
    assert np.all(ks[bt[1, 1]] == ks_prior[bt[1, 1]]) and np.all(ks[bt[1, 1]] > 0)  # kept
    assert np.all(ks[bt[1, 2]] == 0)  # written by zeros only
    assert np.all(ks[bt[2, 0]] == 0) and np.all(ks[bt[2, 1]] == 0)
    ref = r.oracle_decode()
    for kernel, kw in _runs(1, w.head_dim, (dict(), dict(split_tokens=128))):
        out, lse = r.decode(kernel=kernel, **kw)
        r.assert_decode_close(out, lse, ref)


def test_mla_store_all_zero_rows():
    """MLA cache: latent rows and rotary rows that are all zero store scale 0 and codes 0,
    bit-exact with the oracle; the decode over them within the bar."""
    from tests.test_gpu_mla import MlaRun, check_decode, oracle_cache

    w = gen.mla_workload("mla-zero-rows", batch=3, num_heads=16, block_size=16, context_lengths=[20, 65, 1],
                         seed=95, softmax_scale=1.0 / np.sqrt(192.0))
    r = MlaRun(w)
    cu = w.cu_context
    for row in (int(cu[0]) + 3, int(cu[1]) + 64, int(cu[2])):  # 64: sequence 1's new token
        r.t["latent_all"][row].zero_()
    for row in (int(cu[0]) + 3, int(cu[0]) + 19, int(cu[1]) + 10):
        r.t["rope_all"][row].zero_()
    r.store()
    torch.cuda.synchronize()
    hc = oracle_cache(w, r.t)
    assert np.array_equal(r.cache.latent.cpu().numpy(), hc.latent)
    assert np.array_equal(r.cache.rope.cpu().numpy(), hc.rope)
    assert np.array_equal(r.cache.latent_scale.cpu().numpy().view(np.uint32), hc.latent_scale.view(np.uint32))
    assert np.array_equal(r.cache.rope_scale.cpu().numpy().view(np.uint32), hc.rope_scale.view(np.uint32))
    blk, off = w.block_table[1, 64 // 16], 64 % 16
    assert r.cache.latent_scale[blk, off].item() == 0.0
    assert not r.cache.latent[blk, off].any().item()
    for split in (0, 64):
        out, lse = r.decode(split_tokens=split)
        check_decode(r, out, lse, [0, 1, 2], hc=hc)


SCALE_CASES = [
    # mode, D, BS, G, context lengths, q_lens
    (0, 128, 16, 4, [1, 129, 700, 3000], None),
    (1, 128, 16, 5, [20, 300, 2100], [3, 16, 7]),
    (2, 128, 16, 4, [1, 300, 5000], None),
    (3, 64, 32, 8, [33, 500, 1300], None),
]


@pytest.mark.parametrize("mode,d,bs,g,ctx,ql", SCALE_CASES)
def test_softmax_scale_zero_and_negative(mode, d, bs, g, ctx, ql):
    """Scale 0: every visible key weighs the same (the output is the mean of the dequantized values,
    the lse the log of the key count; the oracle is pinned to both).  Negative scales: the query is
    flipped.  Every kernel serving the mode, fixed splits and the balanced partition."""
    r = Run(_wl(mode, d, bs, g, ctx, ql, seed=97 + mode))
    r.store_prior()
    r.store_new()
    for scale in (0.0, -1.0 / np.sqrt(d), -0.7):
        ref = r.oracle_decode(scale=scale)
        if scale == 0.0:  # the lse is the log of each row's key count
            fin = np.isfinite(ref[2])
            counts = np.repeat(r.w.context_lengths if ql is None else
                               np.concatenate([r.w.prior_lengths[b] + 1 + np.arange(r.w.q_lens[b])
                                               for b in range(r.w.batch)]), r.w.num_q_heads).reshape(ref[2].shape)
            assert np.allclose(ref[2][fin], np.log(counts[fin]), rtol=0, atol=1e-12)
        for kernel, kw in _runs(mode, d, (dict(), dict(split_tokens=128), dict(partition=2))):
            out, lse = r.decode(scale=scale, kernel=kernel, **kw)
            r.assert_decode_close(out, lse, ref, scale=scale)


OUTLIER_CASES = [
    # mode, D, BS, G, context lengths, q_lens
    (0, 128, 16, 4, [50, 700, 2500], None),
    (1, 128, 16, 5, [40, 300, 1500], [3, 16, 9]),
    (3, 128, 128, 8, [129, 1000, 3000], None),
    (0, 64, 32, 8, [33, 500], None),
]


@pytest.mark.parametrize("factor", [64, 256])
@pytest.mark.parametrize("mode,d,bs,g,ctx,ql", OUTLIER_CASES)
def test_query_outlier_channels(mode, d, bs, g, ctx, ql, factor):
    """Every query row with one seeded channel multiplied by 64 or 256 (exact in bf16): the logits
    are dominated by that channel and the rest of the row is small beside it.  The int8-score
    kernel rounds each row relative to its largest element; the bar must hold anyway.  All kernels
    that serve the mode, both partitions."""
    w = _wl(mode, d, bs, g, ctx, ql, seed=101 + factor + mode)
    t = gen.gen_tensors(w, device=torch.device("cuda"))
    q = t["q"]
    rng = np.random.default_rng(factor + mode)
    ch = torch.as_tensor(rng.integers(0, d, size=q.shape[:2]), device=q.device)
    mult = torch.ones_like(q, dtype=torch.float32)
    mult.scatter_(2, ch.unsqueeze(2), float(factor))
    t["q"] = (q.float() * mult).to(torch.bfloat16)
    assert torch.equal(t["q"].float(), q.float() * mult)  # a power of two: exact
    r = Run(w, tensors=t)
    r.store_prior()
    r.store_new()
    ref = r.oracle_decode()
    for kernel, kw in _runs(mode, d, (dict(), dict(split_tokens=256), dict(partition=2))):
        out, lse = r.decode(kernel=kernel, **kw)
        max_abs, rel = r.assert_decode_close(out, lse, ref)
        print(f"  outlier x{factor} mode {mode} kernel {kernel} {kw}: max_abs={max_abs:.2e} rel={rel:.2e}")


@pytest.mark.parametrize("factor", [64, 256])
def test_mla_query_outlier_channels(factor):
    """The MLA decode with one latent channel and one rotary channel of every query row multiplied
    by 64 or 256."""
    from tests.test_gpu_mla import MlaRun, check_decode

    w = gen.mla_workload(f"mla-outlier-x{factor}", batch=3, num_heads=16, block_size=64,
                         context_lengths=[100, 1500, 3000], seed=103 + factor, softmax_scale=1.0 / np.sqrt(192.0))
    r = MlaRun(w)
    rng = np.random.default_rng(factor)
    for name, dim in (("q_latent", w.latent_dim), ("q_rope", w.rope_dim)):
        q = r.t[name]
        ch = torch.as_tensor(rng.integers(0, dim, size=q.shape[:2]), device=q.device)
        mult = torch.ones_like(q, dtype=torch.float32)
        mult.scatter_(2, ch.unsqueeze(2), float(factor))
        r.t[name] = (q.float() * mult).to(torch.bfloat16)
    r.store()
    for split in (0, 256):
        out, lse = r.decode(split_tokens=split)
        check_decode(r, out, lse, [0, 1, 2])


def test_decode_on_a_side_stream():
    """A decode launched on another stream, with the output and the workspace allocated by the
    binding: both belong to that stream, so work queued meanwhile on the current stream (here
    allocations filled with NaN) cannot take their memory while the kernels still use it."""
    r = Run(_wl(0, 128, 16, 4, [3000, 1200, 4096, 64, 900], seed=105))
    r.store_prior()
    r.store_new()
    torch.cuda.synchronize()
    ref = r.oracle_decode()
    side = torch.cuda.Stream()  # default priority
    q = r.queries()
    for _ in range(3):
        lse = torch.empty((q.shape[0], r.w.num_q_heads), dtype=torch.float32, device=q.device)
        side.wait_stream(torch.cuda.current_stream())
        out = pkv.decode_gqa(q, r.cache, r.bt, r.ctx, 1.0 / np.sqrt(128), lse_out=lse, stream=side)
        junk = [torch.full((1 << 20,), float("nan"), device=q.device) for _ in range(8)]  # current stream
        del junk
        side.synchronize()
        r.assert_decode_close(out, lse, ref, scale=1.0 / np.sqrt(128))
