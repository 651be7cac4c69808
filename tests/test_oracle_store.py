"""Pins of the oracle's quantizing store (CPU only).

What fixes the store independently of the oracle's own code:
  * hand-worked codes (tests/golden), where halves must go to the even integer;
  * an exhaustive sweep over every finite bf16 value as a token's absmax,
    checked against exact rational arithmetic and the closed-form invariants:
    the absmax element maps to +-127, -128 never occurs, the error is at most
    half a step, codes are odd-symmetric and monotone;
  * the per-block scale equals absmax/127 over every original value the block
    ever received, whatever the order of the chunks.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from gen import custom_workload
from tests.helpers import all_finite_bf16_bits, bits_to_f32, f32_to_bits, nearest_f32, v_token_major

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _store_rows(rows_f32, mode=0, bs=16):
    """Store each row as one token of a one-head cache via slot_mapping; return (codes, scales)."""
    rows = np.asarray(rows_f32, dtype=np.float32)
    t, d = rows.shape
    nb = -(-t // bs)
    cache = oracle.HostCache(mode, nb, 1, bs, d)
    bits = f32_to_bits(rows).reshape(t, 1, d)
    oracle.store(cache, bits, bits, slot_mapping=np.arange(t, dtype=np.int64))
    k = cache.k.reshape(nb * bs, d)[:t].astype(np.int64)
    v = v_token_major(cache.v, bs).reshape(nb * bs, d)[:t].astype(np.int64)
    assert np.array_equal(k, v), "K and V of the same values must quantize identically"
    ks = cache.k_scale.reshape(-1)[:t]
    assert np.array_equal(ks.view(np.uint32), cache.v_scale.reshape(-1)[:t].view(np.uint32))
    return k, ks


def test_golden_per_token_codes():
    spec = json.load(open(os.path.join(GOLDEN, "store_per_token_rne.json")))
    for case in spec["cases"]:
        codes, scales = _store_rows([case["x"]])
        assert scales[0] == np.float32(case["scale"]), case["name"]
        assert codes[0].tolist() == case["codes"], case["name"]


def _sweep_tokens(d=16):
    """Every finite bf16 value v (nonzero) as the absmax of a token; the other entries are
    bf16 values in [-|v|, |v|] drawn from a seeded generator."""
    bits = all_finite_bf16_bits()
    vals = bits_to_f32(bits)
    vals = vals[vals != 0]
    rng = np.random.default_rng(7)
    frac = rng.uniform(-1.0, 1.0, size=(len(vals), d - 1)).astype(np.float32)
    others = (np.abs(vals)[:, None] * frac).astype(np.float32)
    # round the others to bf16 (truncate then fix up: any bf16 value <= |v| will do)
    ob = (others.view(np.uint32) & 0xFFFF0000).view(np.float32)
    rows = np.concatenate([vals[:, None], ob], axis=1)
    return rows


def test_exhaustive_bf16_absmax_sweep_invariants():
    rows = _sweep_tokens()
    codes, scales = _store_rows(rows)
    a = np.abs(rows.astype(np.float64)).max(axis=1)
    # scale is the fp32 absmax/127 (checked exactly on a subset below); here the invariants:
    # (i) the absmax element (column 0) maps to +-127
    assert np.array_equal(np.abs(codes[:, 0]), np.full(len(rows), 127))
    assert np.array_equal(np.sign(codes[:, 0]), np.sign(rows[:, 0]).astype(np.int64))
    # (ii) -128 never occurs
    assert codes.min() >= -127 and codes.max() <= 127
    # (iii) each code is within half a step of x/s (plus the fp32 rounding of the quotient)
    s = scales.astype(np.float64)[:, None]
    ratio = rows.astype(np.float64) / s
    assert np.all(np.abs(codes - ratio) <= 0.5 + 2.0 ** -22 * np.abs(ratio) + 1e-300)
    # the scale is absmax/127 up to fp32 rounding
    assert np.all(np.abs(scales.astype(np.float64) - a / 127.0) <= 2.0 ** -23 * a / 127.0 + 1e-45)


def test_exact_rational_codes_on_sample():
    rows = _sweep_tokens(d=8)
    rng = np.random.default_rng(11)
    pick = rng.choice(len(rows), size=1500, replace=False)
    rows = rows[pick]
    codes, scales = _store_rows(rows)
    for r in range(len(rows)):
        a = max(Fraction(float(abs(x))) for x in rows[r])
        s = nearest_f32(a / 127)
        assert Fraction(float(scales[r])) == s
        for c in range(rows.shape[1]):
            quot = nearest_f32(Fraction(float(rows[r, c])) / s)
            want = max(-128, min(127, round(quot)))  # round() on Fraction: half to even
            assert codes[r, c] == want, (r, c, rows[r, c], float(s))


def test_symmetry_and_monotonicity():
    rows = _sweep_tokens()[::7]
    codes, scales = _store_rows(rows)
    ncodes, nscales = _store_rows(-rows)
    assert np.array_equal(ncodes, -codes)
    assert np.array_equal(nscales, scales)
    order = np.argsort(rows, axis=1, kind="stable")
    sorted_codes = np.take_along_axis(codes, order, axis=1)
    assert np.all(np.diff(sorted_codes, axis=1) >= 0)


def test_per_token_roundtrip_error_bound_random():
    import torch

    w = custom_workload("rt", batch=3, num_q_heads=4, num_kv_heads=2, head_dim=64, block_size=16,
                        quant_mode=0, context_lengths=[5, 40, 17], seed=3)
    g = torch.Generator().manual_seed(5)
    x = (torch.randn(w.total_tokens, 2, 64, generator=g) * 3).to(torch.bfloat16)
    from tests.helpers import torch_bf16_to_bits

    bits = torch_bf16_to_bits(x)
    cache = oracle.HostCache(0, w.num_blocks, 2, 16, 64)
    oracle.store(cache, bits, bits, cu_q_lens=np.r_[0, np.cumsum(w.context_lengths)],
                 context_lengths=w.context_lengths, block_table=w.block_table)
    kd, vd = oracle.dequant(cache, w.block_table, w.context_lengths)
    xf = bits_to_f32(bits).astype(np.float64).reshape(-1, 2, 64)
    for out in (kd, vd):
        y = bits_to_f32(out).astype(np.float64).reshape(-1, 2, 64)
        s = np.abs(xf).max(axis=2, keepdims=True) / 127.0
        # |bf16(q s) - x| <= s/2 (+ quotient rounding) + half a bf16 step of the output
        assert np.all(np.abs(y - xf) <= s * (0.5 + 2.0 ** -17) + np.abs(y) * 2.0 ** -8)


def test_slot_mapping_matches_block_table_form():
    import torch
    from tests.helpers import torch_bf16_to_bits

    w = custom_workload("sm", batch=2, num_q_heads=2, num_kv_heads=2, head_dim=16, block_size=8,
                        quant_mode=0, context_lengths=[9, 20], q_lens=[3, 4], seed=9)
    g = torch.Generator().manual_seed(1)
    x = torch_bf16_to_bits(torch.randn(w.num_new_tokens, 2, 16, generator=g).to(torch.bfloat16))
    c1 = oracle.HostCache(0, w.num_blocks, 2, 8, 16)
    c2 = c1.copy()
    oracle.store(c1, x, x, cu_q_lens=w.cu_q_lens, context_lengths=w.context_lengths,
                 block_table=w.block_table)
    slots = []
    for b in range(w.batch):
        for i in range(int(w.q_lens[b])):
            p = int(w.prior_lengths[b]) + i
            slots.append(int(w.block_table[b, p // 8]) * 8 + p % 8)
    oracle.store(c2, x, x, slot_mapping=np.array(slots, np.int64))
    assert np.array_equal(c1.k, c2.k) and np.array_equal(c1.v, c2.v)
    assert np.array_equal(c1.k_scale, c2.k_scale)
    # a negative slot skips the token
    c3 = oracle.HostCache(0, w.num_blocks, 2, 8, 16)
    oracle.store(c3, x, x, slot_mapping=np.full(len(slots), -1, np.int64))
    assert not c3.k.any() and not c3.k_scale.any()


def test_bf16_mode_is_a_copy():
    import torch
    from tests.helpers import torch_bf16_to_bits

    w = custom_workload("bf", batch=2, num_q_heads=2, num_kv_heads=1, head_dim=32, block_size=16,
                        quant_mode=2, context_lengths=[20, 3], seed=4)
    g = torch.Generator().manual_seed(2)
    x = torch_bf16_to_bits(torch.randn(w.total_tokens, 1, 32, generator=g).to(torch.bfloat16))
    c = oracle.HostCache(2, w.num_blocks, 1, 16, 32)
    oracle.store(c, x, x, cu_q_lens=np.r_[0, np.cumsum(w.context_lengths)],
                 context_lengths=w.context_lengths, block_table=w.block_table)
    kd, vd = oracle.dequant(c, w.block_table, w.context_lengths)
    assert np.array_equal(kd.reshape(x.shape), x) and np.array_equal(vd.reshape(x.shape), x)


# --------------------------------------------------------------------------------------------
# per-block (mode 1)
# --------------------------------------------------------------------------------------------

def _block_store_steps(bs, d, steps, blocks=None):
    """Feed successive chunks of one sequence (one KV head) to the mode-1 store."""
    nblk = max(-(-s["context_length"] // bs) for s in steps)
    bt = np.array([blocks if blocks is not None else list(range(nblk))], np.int32)
    cache = oracle.HostCache(1, bt.max() + 1, 1, bs, d)
    out = []
    for s in steps:
        x = f32_to_bits(np.array(s["new_tokens"], np.float32)).reshape(-1, 1, d)
        n = x.shape[0]
        oracle.store(cache, x, x, cu_q_lens=np.array([0, n], np.int32),
                     context_lengths=np.array([s["context_length"]], np.int32), block_table=bt)
        out.append(cache.copy())
    return bt, out


def test_golden_per_block_rescale():
    spec = json.load(open(os.path.join(GOLDEN, "store_per_block_rescale.json")))
    bs, d = spec["block_size"], spec["head_dim"]
    bt, caches = _block_store_steps(bs, d, spec["steps"])
    for s, c in zip(spec["steps"], caches):
        n = s["context_length"]
        blk = bt[0, 0]
        assert c.k_scale[blk, 0] == np.float32(s["scale"])
        assert c.k[blk, 0, :n].tolist() == s["codes"]
        assert v_token_major(c.v, c.bs)[blk, 0, :n].tolist() == s["codes"]


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_per_block_scale_is_absmax_of_all_originals(seed):
    rng = np.random.default_rng(seed)
    bs, d = 16, 8
    total = int(rng.integers(20, 60))
    # chunk boundaries
    cuts = sorted(set(rng.integers(1, total, size=4).tolist()))
    bounds = [0] + cuts + [total]
    # values grow in magnitude so later chunks force rescales of earlier codes
    x = (rng.standard_normal((total, d)) * np.linspace(0.5, 6.0, total)[:, None]).astype(np.float32)
    xb = (x.view(np.uint32) & 0xFFFF0000).view(np.float32)
    steps = [{"context_length": hi, "new_tokens": xb[lo:hi].tolist()}
             for lo, hi in zip(bounds[:-1], bounds[1:])]
    bt, caches = _block_store_steps(bs, d, steps)
    final = caches[-1]
    for j in range(-(-total // bs)):
        blk = bt[0, j]
        vals = xb[j * bs:min(total, (j + 1) * bs)]
        a = Fraction(float(np.abs(vals).max()))
        assert Fraction(float(final.k_scale[blk, 0])) == nearest_f32(a / 127)
        s = float(final.k_scale[blk, 0])
        codes = final.k[blk, 0, :len(vals)].astype(np.float64)
        # codes never leave [-127, 127]; every value is within one step of its original
        # (half a step when quantized once, up to s_old/2 + s/2 after a rescale)
        assert codes.min() >= -127 and codes.max() <= 127
        assert np.all(np.abs(codes * s - vals) <= s * (1.0 + 2.0 ** -16))
    # tokens of the last chunk were quantized once, under the final scale: half a step
    lo = bounds[-2]
    for p in range(lo, total):
        blk = bt[0, p // bs]
        s = float(final.k_scale[blk, 0])
        code = final.k[blk, 0, p % bs].astype(np.float64)
        assert np.all(np.abs(code * s - xb[p]) <= s * (0.5 + 2.0 ** -16))


def test_per_block_single_chunk_equals_blockwise_absmax_quant():
    rng = np.random.default_rng(5)
    bs, d, total = 16, 8, 37
    x = rng.standard_normal((total, d)).astype(np.float32)
    xb = (x.view(np.uint32) & 0xFFFF0000).view(np.float32)
    bt, caches = _block_store_steps(bs, d, [{"context_length": total, "new_tokens": xb.tolist()}])
    c = caches[0]
    for p in range(total):
        blk = bt[0, p // bs]
        vals = xb[(p // bs) * bs:min(total, (p // bs + 1) * bs)]
        s = nearest_f32(Fraction(float(np.abs(vals).max())) / 127)
        for ch in range(d):
            want = round(nearest_f32(Fraction(float(xb[p, ch])) / s))
            assert c.k[blk, 0, p % bs, ch] == want


def test_per_block_no_growth_keeps_old_codes():
    bs, d = 8, 4
    first = [[4.0, -2.0, 1.0, 0.5], [3.0, 1.0, -4.0, 2.0]]
    second = [[1.0, 1.0, -1.0, 0.25]]  # absmax smaller: scale unchanged
    _, caches = _block_store_steps(bs, d, [{"context_length": 2, "new_tokens": first},
                                           {"context_length": 3, "new_tokens": second}])
    assert np.array_equal(caches[0].k[0, 0, :2], caches[1].k[0, 0, :2])
    assert caches[0].k_scale[0, 0] == caches[1].k_scale[0, 0]


def test_slot_mapping_rejected_for_per_block():
    c = oracle.HostCache(1, 2, 1, 16, 8)
    x = np.zeros((1, 1, 8), np.uint16)
    with pytest.raises(ValueError):
        oracle.store(c, x, x, slot_mapping=np.zeros(1, np.int64))


def test_inactive_decode_slot_stores_nothing():
    """A decode batch slot with context length 0 has no position: its row is ignored and no
    memory outside the live blocks changes."""
    import torch
    from tests.helpers import torch_bf16_to_bits

    w = custom_workload("inactive", batch=3, num_q_heads=2, num_kv_heads=2, head_dim=16, block_size=16,
                        quant_mode=0, context_lengths=[0, 5, 0], seed=2)
    x = torch_bf16_to_bits(torch.randn(3, 2, 16, generator=torch.Generator().manual_seed(0)).to(torch.bfloat16))
    for mode in (0, 1, 2):
        c = oracle.HostCache(mode, w.num_blocks, 2, 16, 16, fill=7)
        ref = c.copy()
        oracle.store(c, x, x, context_lengths=w.context_lengths, block_table=w.block_table)
        blk, slot = w.block_table[1, 0], 4
        # per-token and bf16 modes touch only the new token's slot; the per-block mode may also
        # re-quantize the earlier slots of that block
        ok = (lambda s: s == slot) if mode != 1 else (lambda s: s <= slot)
        changed_k = np.argwhere(c.k != ref.k)
        assert len(changed_k) and all(b == blk and ok(s) for b, _, s, _ in changed_k)
        changed_v = np.argwhere(v_token_major(c.v, c.bs) != v_token_major(ref.v, ref.bs))
        assert len(changed_v) and all(b == blk and ok(s) for b, _, s, _ in changed_v)


def test_per_channel_store_closed_forms():
    """Static per-channel scales (mode 3): codes are clamp(RNE(x / s_c), -128, 127) with s_c the
    channel's own scale, nothing else is written.  Scales are powers of two, so x / s_c is exact and
    every expected code below is written out by hand."""
    d = 8
    # channel c has scale 2^(c - 4); the scale array must come back unchanged
    s = np.array([2.0 ** (c - 4) for c in range(d)], np.float32)
    # multiples of the scale (exact codes), ties (to even), saturation, zero
    mult = np.array([0.0, 1.0, -1.0, 2.5, -2.5, 3.5, 127.5, -129.0], np.float32)
    want = [0, 1, -1, 2, -2, 4, 127, -128]
    mult2 = np.array([126.0, -127.0, 200.0, -200.0, 0.5, -0.5, 1.5, -128.0], np.float32)
    want2 = [126, -127, 127, -128, 0, 0, 2, -128]
    rows = np.stack([mult * s, mult2 * s]).astype(np.float32)  # [2 tokens, d]
    bits = f32_to_bits(rows).reshape(2, 1, d)
    assert np.array_equal(bits_to_f32(bits).reshape(2, d), rows)  # every value is exact in bf16
    c = oracle.HostCache(3, 1, 1, 16, d)
    c.k_scale[0] = s
    c.v_scale[0] = s[::-1]
    oracle.store(c, bits, bits, context_lengths=np.array([2], np.int32), block_table=np.array([[0]], np.int32),
                 cu_q_lens=np.array([0, 2], np.int32))
    assert c.k[0, 0, 0].tolist() == want and c.k[0, 0, 1].tolist() == want2
    assert np.array_equal(c.k_scale[0], s) and np.array_equal(c.v_scale[0], s[::-1])
    # V uses its own (reversed) scales: channel c of V divides by s[d - 1 - c]
    vr = v_token_major(c.v, 16)[0, 0, :2].astype(np.int64)
    exp_v = np.clip(np.rint(rows / s[::-1]), -128, 127).astype(np.int64)  # exact quotients, RNE
    assert np.array_equal(vr, exp_v)
    # a zero scale stores 0 whatever the value
    c.k_scale[0, 3] = 0.0
    c.k[...] = 9
    oracle.store(c, bits, bits, context_lengths=np.array([2], np.int32), block_table=np.array([[0]], np.int32),
                 cu_q_lens=np.array([0, 2], np.int32))
    assert c.k[0, 0, 0, 3] == 0 and c.k[0, 0, 1, 3] == 0


def test_per_channel_codes_depend_on_their_own_channel_scale_only():
    import torch
    from tests.helpers import torch_bf16_to_bits

    rng = np.random.default_rng(3)
    d = 32
    x = torch_bf16_to_bits(torch.randn(4, 1, d, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16))
    base = oracle.HostCache(3, 2, 1, 16, d)
    base.k_scale[0] = rng.uniform(0.005, 0.05, d).astype(np.float32)
    base.v_scale[0] = base.k_scale[0]
    bt = np.array([[1]], np.int32)
    args = dict(context_lengths=np.array([4], np.int32), block_table=bt, cu_q_lens=np.array([0, 4], np.int32))
    c1 = base.copy()
    oracle.store(c1, x, x, **args)
    c2 = base.copy()
    c2.k_scale[0, 7] *= 3
    oracle.store(c2, x, x, **args)
    diff = np.argwhere(c1.k != c2.k)
    assert len(diff) and all(ch == 7 for _, _, _, ch in diff)
