"""Pins of the oracle's fp64 paged attention (CPU only).

Fixed independently of the oracle by:
  * torch's scaled_dot_product_attention in float64 on the gathered,
    contiguous dequantized K/V with enable_gqa (a library routine; its GQA
    convention maps query head h to KV head h // G);
  * closed forms: one key returns that key's value; a zero scale returns the
    mean value; two keys weight as 1 / (1 + exp(l1 - l0)); scipy's logsumexp
    for the log-sum-exp;
  * invariances: the physical placement of blocks and (per-token and bf16
    modes) the block size do not change a single bit; a query never sees keys
    after its own position.
"""
import numpy as np
import pytest

import oracle
from gen import custom_workload
from tests.helpers import bits_to_f32, torch_bf16_to_bits, v_slot


def _build(w, seed=0, kv_scale=1.0):
    """Store K/V for every position of every sequence through the oracle; draw Q."""
    import torch

    g = torch.Generator().manual_seed(seed)
    k = torch_bf16_to_bits((torch.randn(w.total_tokens, w.num_kv_heads, w.head_dim, generator=g)
                            * kv_scale).to(torch.bfloat16))
    v = torch_bf16_to_bits(torch.randn(w.total_tokens, w.num_kv_heads, w.head_dim,
                                       generator=g).to(torch.bfloat16))
    q = torch_bf16_to_bits(torch.randn(w.num_new_tokens, w.num_q_heads, w.head_dim,
                                       generator=g).to(torch.bfloat16))
    c = oracle.HostCache(w.quant_mode, w.num_blocks, w.num_kv_heads, w.block_size, w.head_dim)
    if w.quant_mode == 3:  # static per-channel scales (some values of K saturate)
        rng = np.random.default_rng(seed + 77)
        c.k_scale[...] = rng.uniform(0.01, 0.03, size=c.k_scale.shape).astype(np.float32) * kv_scale
        c.v_scale[...] = rng.uniform(0.01, 0.03, size=c.v_scale.shape).astype(np.float32)
    cu_all = np.zeros(w.batch + 1, np.int32)
    cu_all[1:] = np.cumsum(w.context_lengths)
    if w.quant_mode == 1:
        # per-block scales depend on the chunking: store the prior, then the new tokens
        prior = w.prior_lengths
        pri_idx = np.concatenate([np.arange(cu_all[b], cu_all[b] + prior[b]) for b in range(w.batch)])
        new_idx = np.concatenate([np.arange(cu_all[b] + prior[b], cu_all[b + 1]) for b in range(w.batch)])
        cu_p = np.zeros(w.batch + 1, np.int32)
        cu_p[1:] = np.cumsum(prior)
        oracle.store(c, k[pri_idx], v[pri_idx], cu_q_lens=cu_p, context_lengths=prior,
                     block_table=w.block_table)
        oracle.store(c, k[new_idx], v[new_idx], cu_q_lens=w.cu_q_lens,
                     context_lengths=w.context_lengths, block_table=w.block_table)
    else:
        oracle.store(c, k, v, cu_q_lens=cu_all, context_lengths=w.context_lengths,
                     block_table=w.block_table)
    return c, q, k, v


def _gather_f64(c, w, b, is_v):
    """Dequantized fp64 [ctx, Hkv, D] of sequence b, gathered through the block table."""
    out = np.zeros((int(w.context_lengths[b]), w.num_kv_heads, w.head_dim))
    for p in range(int(w.context_lengths[b])):
        blk, off = w.block_table[b, p // w.block_size], p % w.block_size
        for h in range(w.num_kv_heads):
            if c.mode == 2:
                row = bits_to_f32(v_slot(c.v, blk, h, off, c.bs) if is_v else c.k[blk, h, off]).astype(np.float64)
            else:
                codes = (v_slot(c.v, blk, h, off, c.bs) if is_v else c.k[blk, h, off]).astype(np.float64)
                sc = c.v_scale if is_v else c.k_scale
                if c.mode == 3:
                    s = sc[h].astype(np.float64)
                else:
                    s = float(sc[blk, h, off] if c.mode == 0 else sc[blk, h])
                row = codes * s
            out[p, h] = row
    return out


def _run(c, w, q, scale, nthreads=1, cu=None, window=0):
    return oracle.decode(c, q, w.num_q_heads, w.block_table, w.context_lengths, scale,
                         cu_q_lens=cu if cu is not None else (None if w.decode_only else w.cu_q_lens),
                         nthreads=nthreads, window=window)


@pytest.mark.parametrize("mode,bs,d,g,ctx,ql", [
    (0, 16, 64, 4, [37, 100], None),
    (0, 16, 128, 4, [1, 17, 64, 65], None),
    (0, 128, 128, 8, [300, 129], None),
    (2, 16, 128, 4, [50, 7, 33], None),
    (1, 16, 128, 5, [20, 40, 16], [3, 16, 1]),
    (0, 32, 64, 2, [70, 9], [5, 9]),
    (3, 16, 128, 4, [37, 100, 5], None),
    (3, 128, 64, 8, [300, 129], None),
    (3, 16, 128, 5, [20, 40, 16], [3, 16, 1]),
])
def test_matches_torch_sdpa_fp64(mode, bs, d, g, ctx, ql):
    import torch
    import torch.nn.functional as F

    hkv = 2
    w = custom_workload("p", batch=len(ctx), num_q_heads=hkv * g, num_kv_heads=hkv, head_dim=d,
                        block_size=bs, quant_mode=mode, context_lengths=ctx, q_lens=ql, seed=mode + bs)
    c, q, _, _ = _build(w, seed=d + bs)
    scale = 1.0 / np.sqrt(d)
    out, out64, lse = _run(c, w, q, scale)
    qf = bits_to_f32(q).astype(np.float64)
    cu = w.cu_q_lens
    for b in range(w.batch):
        kk = torch.from_numpy(_gather_f64(c, w, b, False)).permute(1, 0, 2)[None]  # [1, Hkv, n, D]
        vv = torch.from_numpy(_gather_f64(c, w, b, True)).permute(1, 0, 2)[None]
        n = int(w.context_lengths[b])
        qlen = int(w.q_lens[b])
        qq = torch.from_numpy(qf[cu[b]:cu[b] + qlen]).permute(1, 0, 2)[None]  # [1, Hq, qlen, D]
        # causal mask aligned to the end: query i sees keys 0 .. n - qlen + i
        mask = torch.arange(n)[None, :] <= (n - qlen + torch.arange(qlen))[:, None]
        ref = F.scaled_dot_product_attention(qq, kk, vv, attn_mask=mask, scale=scale, enable_gqa=True)
        ref = ref[0].permute(1, 0, 2).numpy()
        got = out64[cu[b]:cu[b] + qlen]
        assert np.allclose(got, ref, rtol=1e-11, atol=1e-12), np.abs(got - ref).max()
        # log-sum-exp against scipy
        from scipy.special import logsumexp

        kr = np.repeat(kk[0].numpy(), g, axis=0)  # [Hq, n, D]
        logits = scale * np.einsum("hqd,hnd->hqn", qq[0].numpy(), kr)
        logits = np.where(mask.numpy()[None], logits, -np.inf)
        want = logsumexp(logits, axis=-1).T  # [qlen, Hq]
        assert np.allclose(lse[cu[b]:cu[b] + qlen], want, rtol=1e-12, atol=1e-12)
    # bf16 output is the fp64 output rounded once
    assert np.array_equal(out, np.vectorize(oracle.bf16_round, otypes=[np.uint16])(out64))


def test_single_key_returns_its_value():
    w = custom_workload("one", batch=3, num_q_heads=8, num_kv_heads=2, head_dim=64, block_size=16,
                        quant_mode=0, context_lengths=[1, 1, 1], seed=1)
    c, q, _, _ = _build(w)
    _, out64, lse = _run(c, w, q, 0.125)
    for b in range(3):
        v0 = _gather_f64(c, w, b, True)[0]  # [Hkv, D]
        assert np.array_equal(out64[b], np.repeat(v0, 4, axis=0))
        k0 = _gather_f64(c, w, b, False)[0]
        qf = bits_to_f32(q[b]).astype(np.float64)
        want = 0.125 * np.einsum("hd,hd->h", qf, np.repeat(k0, 4, axis=0))
        assert np.allclose(lse[b], want, rtol=1e-13, atol=1e-13)


def test_zero_scale_returns_mean_value():
    w = custom_workload("mean", batch=2, num_q_heads=4, num_kv_heads=1, head_dim=32, block_size=16,
                        quant_mode=0, context_lengths=[23, 64], seed=2)
    c, q, _, _ = _build(w)
    _, out64, lse = _run(c, w, q, 0.0)
    for b in range(2):
        mean = _gather_f64(c, w, b, True).mean(axis=0)  # [1, D]
        assert np.allclose(out64[b], np.repeat(mean, 4, axis=0), rtol=1e-12, atol=1e-14)
        assert np.allclose(lse[b], np.log(w.context_lengths[b]), rtol=1e-13)


def test_two_keys_closed_form():
    w = custom_workload("two", batch=1, num_q_heads=2, num_kv_heads=1, head_dim=16, block_size=16,
                        quant_mode=0, context_lengths=[2], seed=3)
    c, q, _, _ = _build(w, seed=8, kv_scale=2.0)
    scale = 0.3
    _, out64, _ = _run(c, w, q, scale)
    k = _gather_f64(c, w, 0, False)[:, 0]
    v = _gather_f64(c, w, 0, True)[:, 0]
    for h in range(2):
        qf = bits_to_f32(q[0, h]).astype(np.float64)
        l0, l1 = scale * qf @ k[0], scale * qf @ k[1]
        w0 = 1.0 / (1.0 + np.exp(l1 - l0))
        assert np.allclose(out64[0, h], w0 * v[0] + (1 - w0) * v[1], rtol=1e-13, atol=1e-14)


def test_empty_sequence_gives_zero_and_minus_inf():
    # a decode batch whose first slot is inactive: ctx 0 (no keys, not even the query's own)
    w = custom_workload("empty", batch=2, num_q_heads=2, num_kv_heads=1, head_dim=16, block_size=16,
                        quant_mode=0, context_lengths=[0, 5], seed=4)
    c, q, _, _ = _build(w)
    qq = np.concatenate([np.zeros((1, 2, 16), np.uint16), q], axis=0)  # one query per sequence
    out, out64, lse = oracle.decode(c, qq, 2, w.block_table, w.context_lengths, 0.25)
    assert np.all(out64[0] == 0) and np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))
    assert np.all(np.isfinite(lse[1]))


@pytest.mark.parametrize("mode", [0, 2, 1])
def test_block_permutation_invariance(mode):
    ctx = [45, 130, 16]
    ql = [1, 1, 1] if mode != 1 else [3, 7, 16]
    w1 = custom_workload("a", batch=3, num_q_heads=8, num_kv_heads=2, head_dim=64, block_size=16,
                         quant_mode=mode, context_lengths=ctx, q_lens=ql, seed=10)
    w2 = custom_workload("b", batch=3, num_q_heads=8, num_kv_heads=2, head_dim=64, block_size=16,
                         quant_mode=mode, context_lengths=ctx, q_lens=ql, seed=99)
    assert not np.array_equal(w1.block_table, w2.block_table)
    c1, q, _, _ = _build(w1, seed=5)
    c2, _, _, _ = _build(w2, seed=5)
    o1 = _run(c1, w1, q, 0.1)
    o2 = _run(c2, w2, q, 0.1)
    for a, b in zip(o1, o2):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("mode", [0, 2])
def test_block_size_invariance(mode):
    ctx = [70, 129]
    outs = []
    for bs in (1, 8, 16, 32, 128):
        w = custom_workload("bs", batch=2, num_q_heads=4, num_kv_heads=2, head_dim=32, block_size=bs,
                            quant_mode=mode, context_lengths=ctx, seed=bs)
        c, q, _, _ = _build(w, seed=6)
        outs.append(_run(c, w, q, 0.2))
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            assert np.array_equal(a, b)


def test_causal_queries_ignore_later_keys():
    w = custom_workload("causal", batch=1, num_q_heads=4, num_kv_heads=1, head_dim=32, block_size=16,
                        quant_mode=0, context_lengths=[40], q_lens=[8], seed=11)
    c, q, _, _ = _build(w, seed=12)
    _, base, _ = _run(c, w, q, 0.2)
    # perturb the key/value at position 35 (query index 3 of the chunk sits at position 35)
    c2 = c.copy()
    blk, off = w.block_table[0, 35 // 16], 35 % 16
    c2.k[blk, 0, off] = -c2.k[blk, 0, off] + 3
    v_slot(c2.v, blk, 0, off, c2.bs)[:] = 100
    _, pert, _ = _run(c2, w, q, 0.2)
    prior = 40 - 8
    for i in range(8):
        same = np.array_equal(base[i], pert[i])
        assert same == (prior + i < 35), i


def test_thread_count_does_not_change_bits():
    w = custom_workload("th", batch=4, num_q_heads=8, num_kv_heads=2, head_dim=64, block_size=16,
                        quant_mode=0, context_lengths=[100, 3, 64, 17], seed=13)
    c, q, _, _ = _build(w, seed=14)
    a = _run(c, w, q, 0.125, nthreads=1)
    b = _run(c, w, q, 0.125, nthreads=5)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_per_channel_with_equal_scales_is_the_per_token_attention():
    """Per-channel scales that are all equal to c give exactly the attention of the per-token mode
    over the same codes with every token scale c (the fp64 values q * c are the same)."""
    w3 = custom_workload("pc", batch=2, num_q_heads=8, num_kv_heads=2, head_dim=64, block_size=16,
                         quant_mode=3, context_lengths=[45, 130], seed=5)
    c3, q, _, _ = _build(w3, seed=9)
    c3.k_scale[...] = np.float32(0.0234375)
    c3.v_scale[...] = np.float32(0.015625)
    w0 = custom_workload("pc", batch=2, num_q_heads=8, num_kv_heads=2, head_dim=64, block_size=16,
                         quant_mode=0, context_lengths=[45, 130], seed=5)
    c0 = oracle.HostCache(0, w0.num_blocks, 2, 16, 64)
    c0.k[...], c0.v[...] = c3.k, c3.v
    c0.k_scale[...] = np.float32(0.0234375)
    c0.v_scale[...] = np.float32(0.015625)
    for a, b in zip(_run(c3, w3, q, 0.125), _run(c0, w0, q, 0.125)):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("mode,bs,d,g,ctx,ql,window", [
    (0, 16, 64, 4, [37, 100, 5], None, 24),
    (1, 16, 128, 5, [20, 40, 16], [3, 16, 1], 7),
    (3, 32, 64, 2, [70, 9], [5, 9], 33),
    (2, 16, 64, 4, [50, 129], None, 64),
])
def test_sliding_window_matches_masked_torch_sdpa(mode, bs, d, g, ctx, ql, window):
    """Sliding window: query at position p sees keys max(0, p - W + 1) .. p; torch's SDPA with that
    boolean mask on the gathered fp64 values is the reference."""
    import torch
    import torch.nn.functional as F

    hkv = 2
    w = custom_workload("sw", batch=len(ctx), num_q_heads=hkv * g, num_kv_heads=hkv, head_dim=d,
                        block_size=bs, quant_mode=mode, context_lengths=ctx, q_lens=ql, seed=mode + bs + 3)
    c, q, _, _ = _build(w, seed=d + bs + 1)
    scale = 1.0 / np.sqrt(d)
    out, out64, lse = _run(c, w, q, scale, window=window)
    qf = bits_to_f32(q).astype(np.float64)
    cu = w.cu_q_lens
    for b in range(w.batch):
        kk = torch.from_numpy(_gather_f64(c, w, b, False)).permute(1, 0, 2)[None]
        vv = torch.from_numpy(_gather_f64(c, w, b, True)).permute(1, 0, 2)[None]
        n = int(w.context_lengths[b])
        qlen = int(w.q_lens[b])
        qq = torch.from_numpy(qf[cu[b]:cu[b] + qlen]).permute(1, 0, 2)[None]
        pos = n - qlen + torch.arange(qlen)[:, None]
        keys = torch.arange(n)[None, :]
        mask = (keys <= pos) & (keys > pos - window)
        ref = F.scaled_dot_product_attention(qq, kk, vv, attn_mask=mask, scale=scale, enable_gqa=True)
        got = out64[cu[b]:cu[b] + qlen]
        assert np.allclose(got, ref[0].permute(1, 0, 2).numpy(), rtol=1e-11, atol=1e-12)


def test_sliding_window_special_cases():
    w = custom_workload("sw2", batch=3, num_q_heads=8, num_kv_heads=2, head_dim=32, block_size=16,
                        quant_mode=0, context_lengths=[45, 130, 1], seed=21)
    c, q, _, _ = _build(w, seed=22)
    base = _run(c, w, q, 0.2)
    # a window at least as long as every context changes nothing, bit for bit
    for a, b in zip(base, _run(c, w, q, 0.2, window=130)):
        assert np.array_equal(a, b)
    # a window of one key: the output is that key's value, the lse its logit
    out, out64, lse = _run(c, w, q, 0.2, window=1)
    qf = bits_to_f32(q).astype(np.float64)
    for b in range(3):
        p = int(w.context_lengths[b]) - 1
        k_self = _gather_f64(c, w, b, False)[p]  # [Hkv, D]
        v_self = _gather_f64(c, w, b, True)[p]
        for hq in range(8):
            assert np.array_equal(out64[b, hq], v_self[hq // 4])
            assert np.isclose(lse[b, hq], 0.2 * float(qf[b, hq] @ k_self[hq // 4]), rtol=1e-13, atol=1e-13)
    # keys before the window do not reach the output
    c2 = c.copy()
    blk = w.block_table[1, 0]
    c2.k[blk] = 100
    v_slot(c2.v, blk, 0, 0, 16)[:] = 100
    v_slot(c2.v, blk, 1, 3, 16)[:] = -100
    for a, b in zip(_run(c, w, q, 0.2, window=100), _run(c2, w, q, 0.2, window=100)):
        assert np.array_equal(a, b)
