"""Pins of the oracle's paged MLA (latent cache) store and decode (CPU only).

The pages list MojoStorePagedMLAKVCache and MojoPagedDecodeMLA (Mojo Opset README, Op List)
without a definition; the oracle reads them as absorbed multi-head latent attention over a
per-token int8 latent row and rotary-key row.  Fixed independently of the oracle by:
  * exact rational arithmetic: every scale is the fp32 nearest to absmax / 127 and every code
    the half-to-even rounding of the fp32 nearest to x / scale, for the latent and the rotary row
    separately, at the slot the block table (or slot mapping) names;
  * torch's scaled_dot_product_attention in float64 with the rotary part concatenated to the
    latent part of query and key and the latent rows as values (every head on one shared KV
    head), and scipy's logsumexp;
  * closed forms (one key, a zero scale, two keys) and invariances (block placement, block
    size, thread count, keys of other sequences).
"""
from fractions import Fraction

import numpy as np
import pytest

import gen
import oracle
from tests.helpers import bits_to_f32, nearest_f32, torch_bf16_to_bits


def _tensors(w, rope_gain=4.0):
    """bf16 bits of the workload's draws; the rotary rows are scaled by a power of two so that
    their scales differ from the latent rows' (exact in bf16)."""
    t = gen.gen_mla_tensors(w)
    t["rope_all"] = t["rope_all"] * rope_gain
    return {k: torch_bf16_to_bits(v) for k, v in t.items()}


def _fill(w, t):
    c = oracle.MLAHostCache(w.num_blocks, w.block_size, w.latent_dim, w.rope_dim)
    cu = np.zeros(w.batch + 1, np.int32)
    cu[1:] = np.cumsum(w.context_lengths)
    oracle.mla_store(c, t["latent_all"], t["rope_all"], cu_q_lens=cu, context_lengths=w.context_lengths,
                     block_table=w.block_table)
    return c


def _gather(c, w, b):
    """fp64 dequantized latent [n, Dc] and rotary [n, Dr] rows of sequence b."""
    n = int(w.context_lengths[b])
    lat = np.zeros((n, w.latent_dim))
    rot = np.zeros((n, w.rope_dim))
    for p in range(n):
        blk, off = w.block_table[b, p // w.block_size], p % w.block_size
        lat[p] = c.latent[blk, off].astype(np.float64) * float(c.latent_scale[blk, off])
        rot[p] = c.rope[blk, off].astype(np.float64) * float(c.rope_scale[blk, off])
    return lat, rot


def _exact_row(x_bits):
    """Scale and codes of one row by exact rational arithmetic."""
    xs = [Fraction(float(v)) for v in bits_to_f32(x_bits)]
    s = nearest_f32(max(abs(v) for v in xs) / 127)
    if s == 0:
        return s, [0] * len(xs)
    return s, [max(-128, min(127, round(nearest_f32(v / s)))) for v in xs]


def test_store_exact_rational_codes_and_slots():
    w = gen.mla_workload("s", batch=3, num_heads=1, block_size=16, context_lengths=[5, 33, 17], seed=3,
                         latent_dim=64, rope_dim=16)
    t = _tensors(w)
    c = _fill(w, t)
    cu = w.cu_context
    for b in range(w.batch):
        for p in range(int(w.context_lengths[b])):
            blk, off = w.block_table[b, p // 16], p % 16
            for codes, scales, src in ((c.latent, c.latent_scale, t["latent_all"]),
                                       (c.rope, c.rope_scale, t["rope_all"])):
                s, want = _exact_row(src[cu[b] + p])
                assert Fraction(float(scales[blk, off])) == s
                assert codes[blk, off].tolist() == want
    # the rotary rows (x4) carry their own, larger scales
    used = w.block_table[w.block_table >= 0]
    assert np.all(c.rope_scale[used][c.rope_scale[used] > 0] > 0)
    assert np.median(c.rope_scale[used]) > 2 * np.median(c.latent_scale[used])


def test_store_absmax_maps_to_127_and_roundtrip_bound():
    w = gen.mla_workload("r", batch=2, num_heads=1, block_size=16, context_lengths=[40, 64], seed=4)
    t = _tensors(w)
    c = _fill(w, t)
    cu = w.cu_context
    for b in range(w.batch):
        for p in range(int(w.context_lengths[b])):
            blk, off = w.block_table[b, p // 16], p % 16
            for codes, scales, src in ((c.latent, c.latent_scale, t["latent_all"]),
                                       (c.rope, c.rope_scale, t["rope_all"])):
                x = bits_to_f32(src[cu[b] + p]).astype(np.float64)
                q = codes[blk, off].astype(np.int64)
                s = float(scales[blk, off])
                i = int(np.argmax(np.abs(x)))
                assert abs(q[i]) == 127 and np.sign(q[i]) == np.sign(x[i])
                assert q.min() >= -127
                assert np.all(np.abs(q * s - x) <= s / 2 * (1 + 2.0 ** -16))


def test_store_slot_mapping_equals_block_table_form_and_skips():
    w = gen.mla_workload("m", batch=2, num_heads=1, block_size=16, context_lengths=[20, 9], seed=5,
                         latent_dim=32, rope_dim=16)
    t = _tensors(w)
    a = _fill(w, t)
    slots = []
    for b in range(w.batch):
        for p in range(int(w.context_lengths[b])):
            slots.append(int(w.block_table[b, p // 16]) * 16 + p % 16)
    # padding tokens (slot -1) interleaved: they are skipped
    n = len(slots)
    sm = np.full(n + 3, -1, np.int64)
    keep = np.sort(np.random.default_rng(0).choice(n + 3, size=n, replace=False))
    sm[keep] = slots
    lat = np.zeros((n + 3, 32), np.uint16)
    rot = np.zeros((n + 3, 16), np.uint16)
    lat[keep], rot[keep] = t["latent_all"], t["rope_all"]
    lat[sm < 0] = 0x3F80  # 1.0: would leave a mark if it were stored
    c = oracle.MLAHostCache(w.num_blocks, 16, 32, 16)
    oracle.mla_store(c, lat, rot, slot_mapping=sm)
    for name in ("latent", "rope", "latent_scale", "rope_scale"):
        assert np.array_equal(getattr(a, name), getattr(c, name))


def test_store_decode_step_writes_only_the_last_position_and_skips_empty():
    w = gen.mla_workload("d", batch=3, num_heads=1, block_size=16, context_lengths=[17, 0, 3], seed=6,
                         latent_dim=32, rope_dim=16, num_blocks=8, max_blocks_per_seq=2)
    t = _tensors(w)
    c = oracle.MLAHostCache(w.num_blocks, 16, 32, 16)
    oracle.mla_store(c, t["latent_all"][:3], t["rope_all"][:3], context_lengths=w.context_lengths,
                     block_table=w.block_table)  # one new token per sequence, no cu_q_lens
    written = np.argwhere(c.latent_scale > 0)
    want = {(int(w.block_table[0, 1]), 0), (int(w.block_table[2, 0]), 2)}
    assert {tuple(x) for x in written} == want
    s, codes = _exact_row(t["latent_all"][2])
    assert c.latent[w.block_table[2, 0], 2].tolist() == codes


@pytest.mark.parametrize("bs,heads,ctx", [(16, 16, [37, 100]), (64, 8, [1, 64, 130]), (32, 32, [70])])
def test_decode_matches_torch_sdpa_fp64(bs, heads, ctx):
    import torch
    import torch.nn.functional as F
    from scipy.special import logsumexp

    w = gen.mla_workload("p", batch=len(ctx), num_heads=heads, block_size=bs, context_lengths=ctx,
                         seed=bs + heads, softmax_scale=1.0 / np.sqrt(192.0))
    t = _tensors(w)
    c = _fill(w, t)
    out, out64, lse = oracle.mla_decode(c, t["q_latent"], t["q_rope"], w.block_table, w.context_lengths,
                                        w.softmax_scale)
    ql = bits_to_f32(t["q_latent"]).astype(np.float64)
    qr = bits_to_f32(t["q_rope"]).astype(np.float64)
    for b in range(w.batch):
        lat, rot = _gather(c, w, b)
        q = torch.from_numpy(np.concatenate([ql[b], qr[b]], axis=1))[None, :, None, :]  # [1, H, 1, 576]
        k = torch.from_numpy(np.concatenate([lat, rot], axis=1))[None, None]  # [1, 1, n, 576]
        v = torch.from_numpy(lat)[None, None]  # [1, 1, n, 512]
        ref = F.scaled_dot_product_attention(q, k, v, scale=w.softmax_scale, enable_gqa=True)[0, :, 0]
        assert np.allclose(out64[b], ref.numpy(), rtol=1e-11, atol=1e-12)
        logits = w.softmax_scale * (ql[b] @ lat.T + qr[b] @ rot.T)  # [H, n]
        assert np.allclose(lse[b], logsumexp(logits, axis=1), rtol=1e-12, atol=1e-12)
    assert np.array_equal(out, np.vectorize(oracle.bf16_round, otypes=[np.uint16])(out64))


def test_decode_closed_forms():
    w = gen.mla_workload("c", batch=3, num_heads=4, block_size=16, context_lengths=[1, 2, 23], seed=7,
                         latent_dim=64, rope_dim=16)
    t = _tensors(w)
    c = _fill(w, t)
    ql = bits_to_f32(t["q_latent"]).astype(np.float64)
    qr = bits_to_f32(t["q_rope"]).astype(np.float64)
    scale = 0.07
    _, out64, lse = oracle.mla_decode(c, t["q_latent"], t["q_rope"], w.block_table, w.context_lengths, scale)
    # one key: its latent row, lse = its logit
    lat, rot = _gather(c, w, 0)
    assert np.array_equal(out64[0], np.repeat(lat, 4, axis=0))
    assert np.allclose(lse[0], scale * (ql[0] @ lat[0] + qr[0] @ rot[0]), rtol=1e-13, atol=1e-13)
    # two keys: weight 1 / (1 + exp(l1 - l0))
    lat, rot = _gather(c, w, 1)
    for h in range(4):
        l0 = scale * (ql[1, h] @ lat[0] + qr[1, h] @ rot[0])
        l1 = scale * (ql[1, h] @ lat[1] + qr[1, h] @ rot[1])
        w0 = 1.0 / (1.0 + np.exp(l1 - l0))
        assert np.allclose(out64[1, h], w0 * lat[0] + (1 - w0) * lat[1], rtol=1e-13, atol=1e-14)
    # zero scale: the mean latent row, lse = ln n
    _, out0, lse0 = oracle.mla_decode(c, t["q_latent"], t["q_rope"], w.block_table, w.context_lengths, 0.0)
    lat, _ = _gather(c, w, 2)
    assert np.allclose(out0[2], np.repeat(lat.mean(axis=0)[None], 4, axis=0), rtol=1e-12, atol=1e-14)
    assert np.allclose(lse0[2], np.log(23.0), rtol=1e-13)


def test_decode_empty_sequence():
    w = gen.mla_workload("e", batch=2, num_heads=2, block_size=16, context_lengths=[0, 5], seed=8,
                         latent_dim=32, rope_dim=16, num_blocks=4, max_blocks_per_seq=1)
    t = _tensors(w)
    c = _fill(w, t)
    out, out64, lse = oracle.mla_decode(c, t["q_latent"], t["q_rope"], w.block_table, w.context_lengths, 0.2)
    assert np.all(out[0] == 0) and np.all(out64[0] == 0) and np.all(np.isneginf(lse[0]))
    assert np.all(np.isfinite(lse[1]))


def test_decode_invariances():
    ctx = [45, 130, 16]
    base = dict(batch=3, num_heads=16, context_lengths=ctx, latent_dim=64, rope_dim=16)
    w1 = gen.mla_workload("a", block_size=16, seed=10, **base)
    w2 = gen.mla_workload("b", block_size=16, seed=99, **base)  # another block placement
    w3 = gen.mla_workload("c", block_size=32, seed=10, **base)  # another block size
    assert not np.array_equal(w1.block_table, w2.block_table)
    t = _tensors(w1)  # same draws for all three (same seed-independent shapes)
    res = []
    for w in (w1, w2, w3):
        c = _fill(w, t)
        res.append(oracle.mla_decode(c, t["q_latent"], t["q_rope"], w.block_table, w.context_lengths, 0.1,
                                     nthreads=1 if w is w1 else 3))
    for r in res[1:]:
        for a, b in zip(res[0], r):
            assert np.array_equal(a, b)
    # a sequence's result does not depend on the other sequences' keys
    c = _fill(w1, t)
    c.latent[w1.block_table[1, :9]] = 77
    r = oracle.mla_decode(c, t["q_latent"], t["q_rope"], w1.block_table, w1.context_lengths, 0.1)
    assert np.array_equal(r[0][0], res[0][0][0]) and np.array_equal(r[0][2], res[0][0][2])
    assert not np.array_equal(r[0][1], res[0][0][1])


def test_decode_rotary_part_counts():
    """Zeroing the rotary query equals SDPA over the latent part alone; the rotary keys then do
    not matter."""
    import torch
    import torch.nn.functional as F

    w = gen.mla_workload("z", batch=1, num_heads=4, block_size=16, context_lengths=[50], seed=11,
                         latent_dim=64, rope_dim=16)
    t = _tensors(w)
    c = _fill(w, t)
    qr0 = np.zeros_like(t["q_rope"])
    _, out64, _ = oracle.mla_decode(c, t["q_latent"], qr0, w.block_table, w.context_lengths, 0.2)
    lat, _ = _gather(c, w, 0)
    q = torch.from_numpy(bits_to_f32(t["q_latent"]).astype(np.float64)[0])[None, :, None, :]
    ref = F.scaled_dot_product_attention(q, torch.from_numpy(lat)[None, None], torch.from_numpy(lat)[None, None],
                                         scale=0.2, enable_gqa=True)[0, :, 0]
    assert np.allclose(out64[0], ref.numpy(), rtol=1e-11, atol=1e-12)
    _, with_rope, _ = oracle.mla_decode(c, t["q_latent"], t["q_rope"], w.block_table, w.context_lengths, 0.2)
    assert not np.allclose(with_rope[0], out64[0], atol=1e-6)
