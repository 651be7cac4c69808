"""Pins of the oracle's bf16 rounding and dequant-gather (CPU only).

Fixed independently of the oracle by: hand-worked products (tests/golden),
exact rational rounding on every finite bf16 grid point and every midpoint,
torch's fp32 -> bf16 cast (a library routine the oracle does not use), and
layout properties (default offsets = exclusive prefix sum, padding rows and
strided outputs untouched).
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from gen import custom_workload
from tests.helpers import all_finite_bf16_bits, bits_to_f32, nearest_bf16, torch_bf16_to_bits, v_slot

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_bf16_round_identity_and_midpoints():
    bits = all_finite_bf16_bits()
    vals = bits_to_f32(bits).astype(np.float64)
    for b, v in zip(bits[::3], vals[::3]):
        assert oracle.bf16_round(v) == int(b) or (v == 0 and oracle.bf16_round(v) in (0, 0x8000))
    # every midpoint between consecutive positive finite bf16 values goes to the even one
    pos = np.sort(vals[(vals > 0)])
    for lo, hi in zip(pos[:-1:5], pos[1::5]):
        mid = (Fraction(float(lo)) + Fraction(float(hi))) / 2
        want = nearest_bf16(mid)
        got = bits_to_f32(np.array([oracle.bf16_round(float(mid))], np.uint16))[0]
        assert Fraction(float(got)) == want
        # just below / above the midpoint go to the nearer neighbour
        below = float(mid) - float(mid) * 2.0 ** -40
        above = float(mid) + float(mid) * 2.0 ** -40
        assert bits_to_f32(np.array([oracle.bf16_round(below)], np.uint16))[0] == lo
        assert bits_to_f32(np.array([oracle.bf16_round(above)], np.uint16))[0] == hi


def test_bf16_round_matches_torch_cast_on_fp32_values():
    import torch

    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 20000),
                        rng.uniform(-1, 1, 5000).astype(np.float32)]).astype(np.float32)
    want = torch_bf16_to_bits(torch.from_numpy(x).to(torch.bfloat16))
    got = np.array([oracle.bf16_round(float(v)) for v in x], np.uint16)
    assert np.array_equal(got, want)


def test_bf16_round_fp64_single_rounding():
    # values that an fp64 -> fp32 -> bf16 chain would double-round
    for base in (1.0, 3.0, 1.0e-3, 7.5e10):
        e = np.floor(np.log2(base))
        step = 2.0 ** (e - 7)
        v = base + step / 2 + step * 2.0 ** -30  # just above a midpoint, within fp32's lost bits
        got = Fraction(float(bits_to_f32(np.array([oracle.bf16_round(v)], np.uint16))[0]))
        assert got == nearest_bf16(Fraction(v))


def test_golden_dequant_products():
    spec = json.load(open(os.path.join(GOLDEN, "dequant_bf16_rne.json")))
    for case in spec["cases"]:
        c = oracle.HostCache(0, 1, 1, 16, 1)
        c.k[0, 0, 0, 0] = case["code"]
        v_slot(c.v, 0, 0, 0, 16)[0] = case["code"]
        c.k_scale[0, 0, 0] = case["scale"]
        c.v_scale[0, 0, 0] = case["scale"]
        k, v = oracle.dequant(c, np.array([[0]], np.int32), np.array([1], np.int32))
        assert int(k[0]) == int(case["bf16_bits"], 16), case["note"]
        assert int(v[0]) == int(case["bf16_bits"], 16), case["note"]


def _random_cache(mode, w, seed):
    rng = np.random.default_rng(seed)
    c = oracle.HostCache(mode, w.num_blocks, w.num_kv_heads, w.block_size, w.head_dim)
    if mode == 2:
        import torch

        g = torch.Generator().manual_seed(seed)
        c.k[...] = torch_bf16_to_bits(torch.randn(c.k.shape, generator=g).to(torch.bfloat16))
        c.v[...] = torch_bf16_to_bits(torch.randn(c.v.shape, generator=g).to(torch.bfloat16))
    else:
        c.k[...] = rng.integers(-127, 128, size=c.k.shape)
        c.v[...] = rng.integers(-127, 128, size=c.v.shape)
        c.k_scale[...] = rng.uniform(1e-3, 0.1, size=c.k_scale.shape).astype(np.float32)
        c.v_scale[...] = rng.uniform(1e-3, 0.1, size=c.v_scale.shape).astype(np.float32)
    return c


@pytest.mark.parametrize("mode", [0, 1, 2, 3])
def test_dequant_matches_torch_fp32_product(mode):
    """Gather by hand with numpy indexing, multiply in fp32 and cast with torch."""
    import torch

    w = custom_workload("dq", batch=3, num_q_heads=4, num_kv_heads=2, head_dim=32, block_size=16,
                        quant_mode=mode, context_lengths=[1, 33, 64], seed=mode)
    c = _random_cache(mode, w, 10 + mode)
    kd, vd = oracle.dequant(c, w.block_table, w.context_lengths)
    kd = kd.reshape(-1, 2, 32)
    vd = vd.reshape(-1, 2, 32)
    row = 0
    for b in range(w.batch):
        for p in range(int(w.context_lengths[b])):
            blk, off = w.block_table[b, p // 16], p % 16
            for h in range(2):
                if mode == 2:
                    wk, wv = c.k[blk, h, off], v_slot(c.v, blk, h, off, 16)
                else:
                    if mode == 3:  # one scale per channel: a vector over the row
                        sk, sv = torch.from_numpy(c.k_scale[h]), torch.from_numpy(c.v_scale[h])
                    else:
                        sk = torch.tensor(c.k_scale[blk, h, off] if mode == 0 else c.k_scale[blk, h])
                        sv = torch.tensor(c.v_scale[blk, h, off] if mode == 0 else c.v_scale[blk, h])
                    tk = torch.from_numpy(c.k[blk, h, off].astype(np.float32)) * sk
                    tv = torch.from_numpy(v_slot(c.v, blk, h, off, 16).astype(np.float32)) * sv
                    wk = torch_bf16_to_bits(tk.to(torch.bfloat16))
                    wv = torch_bf16_to_bits(tv.to(torch.bfloat16))
                assert np.array_equal(kd[row, h], wk)
                assert np.array_equal(vd[row, h], wv)
            row += 1


def test_dequant_offsets_padding_and_strides():
    w = custom_workload("dq2", batch=3, num_q_heads=2, num_kv_heads=2, head_dim=16, block_size=16,
                        quant_mode=0, context_lengths=[5, 0, 20], seed=3)
    c = _random_cache(0, w, 4)
    packed_k, packed_v = oracle.dequant(c, w.block_table, w.context_lengths)
    # padded layout: each sequence starts at a caller offset; head-major strided rows
    pad = np.array([3, 7, 2])
    offs = np.zeros(3, np.int64)
    offs[1:] = np.cumsum(w.context_lengths + pad)[:-1]
    rows = int((offs + w.context_lengths + pad).max())
    token_stride, head_stride = 16, rows * 16  # [Hkv][rows][D] layout
    sentinel = 0xDEAD
    ko = np.full(rows * 2 * 16, sentinel, np.uint16)
    vo = np.full(rows * 2 * 16, sentinel, np.uint16)
    oracle.dequant(c, w.block_table, w.context_lengths, seq_offsets=offs, k_out=ko, v_out=vo,
                   token_stride=token_stride, head_stride=head_stride)
    ko = ko.reshape(2, rows, 16)
    pk = packed_k.reshape(-1, 2, 16)
    written = np.zeros(rows, bool)
    src = 0
    for b in range(3):
        n = int(w.context_lengths[b])
        for p in range(n):
            assert np.array_equal(ko[:, offs[b] + p, :], pk[src + p])
            written[offs[b] + p] = True
        src += n
    assert np.all(ko[:, ~written, :] == sentinel)
