"""GPU parity: libpkv (through the C ABI) against the CPU oracle on the same seeded inputs.

Bars: int8 codes and fp32 scales bit-exact; dequant bit-exact; attention within max-abs 1e-2 and
norm-relative 1e-2 of the oracle's fp64 result (elementwise |g - o| <= 1e-2 + 1e-2 |o|); lse within
1e-4 + 1e-5 |lse| plus the error bound of an fp32 evaluation of the logits (gpu_harness.lse_bar).
Sizes span several 128-key chunks, several splits and ragged tails.
"""
import numpy as np
import pytest
import torch

import gen
import oracle
import paged_kv_cache_c8_amd as pkv
from tests.gpu_harness import Run, bits, i32
from tests.helpers import v_token_major

pytestmark = pytest.mark.gpu


def _wl(mode, d, bs, g, ctx, ql=None, hkv=2, seed=0, **kw):
    return gen.custom_workload(f"m{mode}-d{d}-bs{bs}-g{g}", batch=len(ctx), num_q_heads=hkv * g,
                               num_kv_heads=hkv, head_dim=d, block_size=bs, quant_mode=mode,
                               context_lengths=ctx, q_lens=ql, seed=seed, **kw)


def test_tiny_config_end_to_end():
    r = Run(gen.make_config(0))
    r.store_prior()
    r.store_new()
    r.assert_cache_equal()
    out, lse = r.decode()
    r.assert_decode_close(out, lse)


DECODE_CASES = [
    # mode, D, BS, G, context lengths
    (0, 128, 16, 4, [1, 2, 15, 16, 17, 127, 128, 129, 300, 1000]),
    (0, 128, 128, 8, [1, 129, 257, 700, 1500]),
    (0, 64, 16, 4, [37, 100, 5, 260]),
    (0, 64, 32, 8, [33, 64, 65, 500]),
    (0, 128, 64, 2, [63, 64, 65, 900]),
    (0, 128, 16, 1, [50, 333]),
    (0, 128, 16, 5, [40, 257, 129]),
    (0, 128, 16, 16, [77, 600]),
    (2, 128, 16, 4, [1, 16, 17, 129, 513]),
    (2, 64, 128, 8, [200, 1, 129]),
    (1, 128, 16, 4, [20, 129, 300]),
    (1, 64, 64, 8, [65, 1, 200]),
    # more than 16 query heads per KV head: two 16-row groups sharing each key block (the second
    # one partly filled), per token and per block
    (0, 128, 16, 32, [300, 1025, 1]),
    (1, 64, 16, 24, [70, 500]),
]


KERNELS = [1, 2, 3]  # VALU split-KV kernel, MFMA kernel (fp16 scores), MFMA kernel (int8 scores)


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("mode,d,bs,g,ctx", DECODE_CASES)
def test_decode_matches_oracle(mode, d, bs, g, ctx, kernel):
    r = Run(_wl(mode, d, bs, g, ctx, seed=len(ctx) + d + bs + g))
    r.store_prior()
    r.store_new()
    r.assert_cache_equal()
    out, lse = r.decode(kernel=kernel)
    ref = r.oracle_decode()
    r.assert_decode_close(out, lse, ref)
    # several partitions of the keys: the same result within rounding
    for split in (128, 256):
        o2, l2 = r.decode(split_tokens=split, kernel=kernel)
        r.assert_decode_close(o2, l2, ref)


CHUNK_CASES = [
    # mode, D, BS, G, context lengths, q_lens
    (1, 128, 16, 5, [20, 40, 16, 300], [3, 16, 1, 7]),
    (1, 128, 16, 4, [1, 17, 33, 129], [1, 16, 2, 9]),
    (0, 128, 16, 4, [70, 9, 200], [5, 9, 16]),
    (0, 64, 32, 2, [300, 31], [12, 31]),
    (2, 128, 16, 8, [50, 129], [4, 13]),
    # three KV heads x three sequences: pairs of (split, sequence x KV head) not a multiple of 8,
    # up to five 16-row groups each (the workgroup order puts a pair's row groups 8 apart)
    (1, 128, 16, 5, [500, 37, 260], [16, 11, 6], 3),
    # six 16-row groups of one (sequence, KV head) sharing their keys, static per-channel scales;
    # a short sequence whose later row groups hold no rows
    (3, 128, 32, 6, [100, 1000, 3], [16, 16, 3]),
]


PREFILL_CASES = [
    # mode, D, BS, G, context lengths, q_lens: whole prompts (prior 0) and long chunks after a prior
    (0, 128, 16, 4, [512, 300], [512, 300]),
    (1, 128, 16, 5, [1200, 700], [400, 700]),
    (3, 128, 128, 8, [1000, 129], [600, 129]),
    (0, 64, 64, 2, [777, 1], [777, 1]),
    (2, 128, 16, 4, [700, 250], [350, 250]),
]


@pytest.mark.parametrize("mode,d,bs,g,ctx,ql", PREFILL_CASES)
def test_paged_prefill_matches_oracle(mode, d, bs, g, ctx, ql):
    """Paged prefill (MojoPagedPrefillGQA, Mojo Opset README Op List): hundreds of causal queries per sequence through the same
    kernels (many row groups per KV head), against the oracle; also with fixed splits."""
    r = Run(_wl(mode, d, bs, g, ctx, ql, seed=sum(ctx) + mode))
    r.store_prior()
    r.store_new()
    r.assert_cache_equal()
    ref = r.oracle_decode(nthreads=16)
    out, lse = r.decode()
    r.assert_decode_close(out, lse, ref)
    o2, l2 = r.decode(split_tokens=256)
    r.assert_decode_close(o2, l2, ref)


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("case", CHUNK_CASES)
def test_chunked_store_and_causal_decode(case, kernel):
    mode, d, bs, g, ctx, ql = case[:6]
    hkv = case[6] if len(case) > 6 else 2
    if mode == 3 and kernel != 3:
        pytest.skip("static per-channel scales are decoded by the int8-score kernel only")
    r = Run(_wl(mode, d, bs, g, ctx, ql, hkv=hkv, seed=sum(ctx)))
    r.store_prior()
    r.store_new()
    r.assert_cache_equal()
    out, lse = r.decode(kernel=kernel)
    ref = r.oracle_decode()
    r.assert_decode_close(out, lse, ref)
    o2, l2 = r.decode(split_tokens=128, kernel=kernel)
    r.assert_decode_close(o2, l2, ref)


@pytest.mark.parametrize("kernel", KERNELS)
def test_split_count_agreement_and_determinism(kernel):
    r = Run(_wl(0, 128, 16, 4, [3000, 1200, 4096, 64], seed=5), with_oracle=False)
    r.store_prior()
    r.store_new()
    one, l1 = r.decode(split_tokens=4096, kernel=kernel)
    many, lm = r.decode(split_tokens=128, kernel=kernel)
    default, ld = r.decode(kernel=kernel)
    default2, ld2 = r.decode(kernel=kernel)
    torch.cuda.synchronize()
    assert torch.equal(default.view(torch.int16), default2.view(torch.int16))
    assert torch.equal(ld, ld2)
    # Partitions differ only in rounding: the softmax weights enter the P.V dot products as fp16
    # (relative rounding <= 2^-11, dependent on the running max and so on the split boundaries)
    # and the output is rounded to bf16 (one step <= 2^-7 relative).  The lse is all fp32.
    for o, l in ((many, lm), (default, ld)):
        diff = (o.float() - one.float()).abs()
        bound = one.float().abs() * 2.0 ** -7 + 2.0 ** -10 * float(one.float().abs().max())
        assert bool((diff <= bound).all()), float((diff - bound).max())
        assert torch.allclose(l, l1, rtol=1e-5, atol=1e-5)


def test_block_permutation_invariance_on_gpu():
    ctx = [700, 45, 1300]
    w1 = _wl(0, 128, 16, 4, ctx, seed=1)
    w2 = _wl(0, 128, 16, 4, ctx, seed=2)
    assert not np.array_equal(w1.block_table, w2.block_table)
    r1 = Run(w1, with_oracle=False)
    r2 = Run(w2, with_oracle=False, tensors=r1.t)
    for r in (r1, r2):
        r.store_prior()
        r.store_new()
    o1, l1 = r1.decode()
    o2, l2 = r2.decode()
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


@pytest.mark.parametrize("kernel", KERNELS)
def test_inactive_sequences_give_zero_and_minus_inf(kernel):
    r = Run(_wl(0, 128, 16, 4, [0, 50, 0, 300], seed=3))
    r.store_prior()
    r.store_new()
    r.assert_cache_equal()
    for split in (0, 128):
        out, lse = r.decode(split_tokens=split, kernel=kernel)
        torch.cuda.synchronize()
        assert bool((out[0] == 0).all()) and bool((out[2] == 0).all())
        assert bool(torch.isneginf(lse[0]).all()) and bool(torch.isneginf(lse[2]).all())
        r.assert_decode_close(out, lse)


@pytest.mark.parametrize("d", [64, 128])
def test_exhaustive_bf16_sweep_through_store(d):
    """Every finite bf16 value as the absmax of one token (others: seeded values below it); the
    two zeros give all-zero tokens (scale 0, codes 0)."""
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    b = b[((b >> 7) & 0xFF) != 0xFF]
    vals = (b.astype(np.uint32) << 16).view(np.float32)
    rng = np.random.default_rng(d)
    frac = rng.uniform(-1, 1, size=(len(vals), d - 1)).astype(np.float32)
    others = ((np.abs(vals)[:, None] * frac).view(np.uint32) & 0xFFFF0000).view(np.float32)
    rows = np.concatenate([vals[:, None], others], axis=1)
    rows_bits = (rows.view(np.uint32) >> 16).astype(np.uint16).reshape(-1, 1, d)
    t = len(rows)
    bs = 16
    nb = -(-t // bs)
    dev = torch.device("cuda")
    x = torch.from_numpy(rows_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    cache = pkv.Cache(0, nb, 1, bs, d, device=dev)
    slots = torch.arange(t, dtype=torch.int64, device=dev)
    pkv.store_c8(cache, x, x, slot_mapping=slots)
    hc = oracle.HostCache(0, nb, 1, bs, d)
    oracle.store(hc, rows_bits, rows_bits, slot_mapping=np.arange(t, dtype=np.int64))
    torch.cuda.synchronize()
    assert np.array_equal(cache.k.cpu().numpy(), hc.k)
    assert np.array_equal(cache.v.cpu().numpy(), hc.v)
    assert np.array_equal(cache.k_scale.cpu().numpy().view(np.uint32), hc.k_scale.view(np.uint32))
    assert np.array_equal(cache.v_scale.cpu().numpy().view(np.uint32), hc.v_scale.view(np.uint32))
    zero = np.flatnonzero(vals == 0)  # +0 and -0: scale 0 and every code 0
    assert len(zero) == 2 and np.all(hc.k_scale.reshape(-1)[zero] == 0)
    assert np.all(cache.k.cpu().numpy().reshape(-1, d)[:t][zero] == 0)
    # the same rows as one prompt of a single sequence (the 16-slot tile kernel), and split into
    # ragged chunks of several sequences (tiles the call fills in part)
    bt = torch.arange(nb, dtype=torch.int32, device=dev).view(1, nb)
    for lens in ([t], [5, 700, t - 705]):
        cache2 = pkv.Cache(0, nb, 1, bs, d, device=dev)
        cache2.v.fill_(77)  # slots of a partly filled tile keep what they held
        done = 0
        for n in lens:
            pkv.store_c8(cache2, x[done:done + n], x[done:done + n], cu_q_lens=torch.tensor([0, n], dtype=torch.int32, device=dev),
                         context_lengths=torch.tensor([done + n], dtype=torch.int32, device=dev), block_table=bt,
                         max_q_len=n)
            done += n
        torch.cuda.synchronize()
        assert np.array_equal(cache2.k.cpu().numpy(), hc.k)
        assert np.array_equal(cache2.k_scale.cpu().numpy().view(np.uint32), hc.k_scale.view(np.uint32))
        assert np.array_equal(cache2.v_scale.cpu().numpy().view(np.uint32), hc.v_scale.view(np.uint32))
        vt = v_token_major(cache2.v.cpu().numpy(), bs).reshape(-1, d)[:t]
        assert np.array_equal(vt, v_token_major(hc.v, bs).reshape(-1, d)[:t])


def test_slot_mapping_store_with_skips():
    dev = torch.device("cuda")
    w = _wl(0, 128, 32, 4, [10, 70], seed=8)
    t = gen.gen_tensors(w, device=dev)
    n = w.total_tokens
    rng = np.random.default_rng(0)
    slots = rng.permutation(w.num_blocks * w.block_size)[:n].astype(np.int64)
    slots[::7] = -1
    cache = pkv.Cache(0, w.num_blocks, 2, 32, 128, device=dev)
    pkv.store_c8(cache, t["k_all"], t["v_all"], slot_mapping=torch.as_tensor(slots, device=dev))
    hc = oracle.HostCache(0, w.num_blocks, 2, 32, 128)
    oracle.store(hc, bits(t["k_all"]), bits(t["v_all"]), slot_mapping=slots)
    torch.cuda.synchronize()
    assert np.array_equal(cache.k.cpu().numpy(), hc.k)
    assert np.array_equal(cache.v.cpu().numpy(), hc.v)
    assert np.array_equal(cache.k_scale.cpu().numpy().view(np.uint32), hc.k_scale.view(np.uint32))


@pytest.mark.parametrize("mode,d,bs", [(0, 128, 16), (1, 128, 16), (2, 128, 16), (0, 64, 128),
                                       (1, 64, 32), (2, 64, 64), (3, 128, 16), (3, 64, 128)])
def test_dequant_bit_exact(mode, d, bs):
    ql = [1, 5, 16] if mode == 1 else None
    w = _wl(mode, d, bs, 2, [1, 40, 300], ql, seed=d + bs)
    r = Run(w)
    r.store_prior()
    r.store_new()
    k, v = pkv.dequant(r.cache, r.bt, r.ctx)
    ko, vo = oracle.dequant(r.hc, w.block_table, w.context_lengths)
    torch.cuda.synchronize()
    assert np.array_equal(bits(k).reshape(-1), ko[:k.numel()])
    assert np.array_equal(bits(v).reshape(-1), vo[:v.numel()])


def test_dequant_padded_offsets_and_strides():
    w = _wl(0, 128, 16, 2, [5, 0, 40, 17], seed=4)
    r = Run(w)
    r.store_prior()
    r.store_new()
    pad = np.array([3, 7, 2, 5])
    offs = np.zeros(4, np.int64)
    offs[1:] = np.cumsum(w.context_lengths + pad)[:-1]
    rows = int((offs + w.context_lengths + pad).max())
    hkv, d = 2, 128
    for token_stride, head_stride in ((d, rows * d), (hkv * d + 8, d), (hkv * d + 3, d + 1)):
        n = rows * max(token_stride, 1) + hkv * head_stride + d
        kd = torch.full((n,), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)
        vd = torch.full((n,), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)
        pkv.dequant(r.cache, r.bt, r.ctx, seq_offsets=torch.as_tensor(offs, device="cuda"), k_out=kd,
                    v_out=vd, token_stride=token_stride, head_stride=head_stride)
        ko = np.full(n, 0xFFFF, np.uint16)
        vo = np.full(n, 0xFFFF, np.uint16)
        oracle.dequant(r.hc, w.block_table, w.context_lengths, seq_offsets=offs, k_out=ko, v_out=vo,
                       token_stride=token_stride, head_stride=head_stride)
        torch.cuda.synchronize()
        assert np.array_equal(bits(kd), ko)
        assert np.array_equal(bits(vd), vo)


def test_per_block_rescale_sequence_matches_oracle():
    """Several chunk stores into the same blocks (scales grow, codes re-quantized)."""
    dev = torch.device("cuda")
    bs, d, hkv = 16, 128, 2
    steps = [(0, 5), (5, 9), (9, 30), (30, 31), (31, 64)]
    total = steps[-1][1]
    bt = np.array([[3, 0, 2, 1]], np.int32)
    g = torch.Generator(device=dev).manual_seed(3)
    growth = torch.linspace(0.5, 8.0, total, device=dev)[:, None, None]
    x = (torch.randn(total, hkv, d, generator=g, device=dev) * growth).to(torch.bfloat16)
    cache = pkv.Cache(1, 4, hkv, bs, d, device=dev)
    hc = oracle.HostCache(1, 4, hkv, bs, d)
    for lo, hi in steps:
        cu = np.array([0, hi - lo], np.int32)
        ctx = np.array([hi], np.int32)
        pkv.store_c8(cache, x[lo:hi], x[lo:hi], cu_q_lens=i32(cu, dev), context_lengths=i32(ctx, dev),
                     block_table=i32(bt, dev), max_q_len=hi - lo)
        oracle.store(hc, bits(x[lo:hi]), bits(x[lo:hi]), cu_q_lens=cu, context_lengths=ctx, block_table=bt)
        torch.cuda.synchronize()
        assert np.array_equal(cache.k.cpu().numpy(), hc.k), (lo, hi)
        assert np.array_equal(cache.v.cpu().numpy(), hc.v), (lo, hi)
        assert np.array_equal(cache.k_scale.cpu().numpy().view(np.uint32), hc.k_scale.view(np.uint32))


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("mode", [0, 1, 2])
def test_unwritten_slots_do_not_reach_the_output(mode, kernel):
    """Slots past each sequence's keys hold whatever the pool held before (here NaN scales, NaN
    bf16 values or the largest code): the decode reads them only as in-bounds stand-ins and must
    give them zero weight."""
    w = _wl(mode, 128, 16, 4, [1, 17, 100, 531], seed=77)
    r = Run(w)
    if mode == 2:
        r.cache.k.fill_(float("nan"))
        r.cache.v.fill_(float("nan"))
    else:
        r.cache.k.fill_(127)
        r.cache.v.fill_(127)
        r.cache.k_scale.fill_(float("nan"))
        r.cache.v_scale.fill_(float("nan"))
    r.store_prior()
    r.store_new()
    out, lse = r.decode(kernel=kernel)
    assert torch.isfinite(out.float()).all()
    r.assert_decode_close(out, lse)


def test_balanced_partition_edge_cases():
    """The planned (balanced) partition of the int8-score kernel: a batch with no key at all, a
    batch mixing one-block and long sequences (one-segment and many-segment items), a multi-token
    batch (one subset class, two row tiles), a batch of many short sequences, and more sequences
    than the balanced partition takes (the fixed-split plan is used)."""
    # every sequence empty: only the merge writes (zero rows, lse -inf)
    r = Run(_wl(0, 128, 16, 4, [0, 0, 0], seed=11))
    r.store_prior()
    r.store_new()
    out, lse = r.decode(partition=2)
    torch.cuda.synchronize()
    assert bool((out == 0).all()) and bool(torch.isneginf(lse).all())
    # short and long sequences together
    r = Run(_wl(0, 128, 16, 4, [1, 5, 64, 65, 2000, 3, 4096, 700], seed=12))
    r.store_prior()
    r.store_new()
    out, lse = r.decode(partition=2)
    r.assert_decode_close(out, lse)
    # multi-token rows: 16 x 5 = 80 rows per KV head (two 16-row tiles per row group)
    r = Run(_wl(1, 128, 16, 5, [40, 700, 17, 1500], [16, 9, 16, 3], seed=13))
    r.store_prior()
    r.store_new()
    out, lse = r.decode(partition=2)
    r.assert_decode_close(out, lse)
    # 600 sequences x 8 KV heads, then 4200 sequences: beyond the balanced partition's limit of
    # 4096 sequences (the fixed-split plan is used)
    ctx = list(np.random.default_rng(14).integers(0, 40, size=600))
    r = Run(_wl(0, 64, 16, 4, ctx, hkv=8, seed=14))
    r.store_prior()
    r.store_new()
    out, lse = r.decode(partition=2)
    r.assert_decode_close(out, lse)
    ctx = list(np.random.default_rng(16).integers(0, 20, size=4200))
    r = Run(_wl(0, 64, 16, 4, ctx, hkv=2, seed=16))
    r.store_prior()
    r.store_new()
    out, lse = r.decode(partition=2)
    r.assert_decode_close(out, lse)


def test_bf16_balanced_partition():
    """The balanced partition of the bf16 matrix-core kernel (segments over several rounds of the
    GPU's waves; segments longer than one 4096-key range are walked range by range): empty
    batches, one-block and long sequences together, three KV heads of eight query heads, a
    sliding window, agreement with fixed splits and between repeated calls, and head_dim 64."""
    r = Run(_wl(2, 128, 16, 4, [0, 0, 0], seed=41))
    r.store_prior()
    r.store_new()
    out, lse = r.decode(partition=2)
    torch.cuda.synchronize()
    assert bool((out == 0).all()) and bool(torch.isneginf(lse).all())
    r = Run(_wl(2, 128, 16, 4, [1, 5, 64, 65, 9000, 3, 4096, 700, 0, 12000], seed=42))
    r.store_prior()
    r.store_new()
    plan = pkv.decode_plan(r.w.batch, r.w.num_q_heads, r.w.num_kv_heads, 128, r.w.max_blocks_per_seq, 16, 1, 2,
                           partition=2)
    assert plan["split_tokens"] == 0 and plan["num_splits"] > 0, plan
    out, lse = r.decode(partition=2)
    r.assert_decode_close(out, lse)
    again, lse2 = r.decode(partition=2)
    fixed, lf = r.decode(split_tokens=4096)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), again.view(torch.int16)) and torch.equal(lse, lse2)
    diff = (out.float() - fixed.float()).abs()
    bound = fixed.float().abs() * 2.0 ** -7 + 2.0 ** -10 * float(fixed.float().abs().max())
    assert bool((diff <= bound).all()), float((diff - bound).max())
    fin = torch.isfinite(lf)
    assert torch.equal(fin, torch.isfinite(lse)) and torch.allclose(lse[fin], lf[fin], rtol=1e-5, atol=1e-5)
    r = Run(_wl(2, 128, 32, 8, [300, 5000, 33, 2048], hkv=3, seed=43))
    r.store_prior()
    r.store_new()
    out, lse = r.decode(partition=2)
    r.assert_decode_close(out, lse)
    out, lse = r.decode(partition=2, window=700)
    r.assert_decode_close(out, lse, r.oracle_decode(window=700))
    # head_dim 64: every output channel (its last channel tile once came out wrong beside a right
    # lse), one-segment and many-segment items, against the oracle and against fixed splits
    r = Run(_wl(2, 64, 32, 8, [300, 5000, 33, 2048], hkv=3, seed=44))
    r.store_prior()
    r.store_new()
    assert pkv.decode_plan(r.w.batch, r.w.num_q_heads, 3, 64, r.w.max_blocks_per_seq, 32, 1, 2,
                           partition=2)["split_tokens"] == 0
    out, lse = r.decode(partition=2)
    r.assert_decode_close(out, lse)
    fixed, _ = r.decode(split_tokens=512)
    torch.cuda.synchronize()
    diff = (out.float() - fixed.float()).abs()
    bound = fixed.float().abs() * 2.0 ** -7 + 2.0 ** -10 * float(fixed.float().abs().max())
    assert bool((diff <= bound).all()), float((diff - bound).max())


@pytest.mark.parametrize("mode,g,bs,ctx", [(0, 8, 32, [33, 4097, 65]), (3, 8, 32, [33, 1000, 65]),
                                             (0, 4, 16, [33, 4097, 65]), (1, 4, 16, [5000, 3000]),
                                             (0, 8, 32, [600, 4097])])
def test_balanced_partition_head_dim_64(mode, g, bs, ctx):
    """The int8-score kernel's balanced partition at head_dim 64 with items of one and of many
    segments (their partials merged by several thread groups): every output channel within the bar,
    not only the lse (wrong outputs beside a right lse have been seen here)."""
    r = Run(_wl(mode, 64, bs, g, ctx, seed=sum(ctx) + g + mode))
    r.store_prior()
    r.store_new()
    plan = pkv.decode_plan(r.w.batch, r.w.num_q_heads, 2, 64, r.w.max_blocks_per_seq, bs, 1, mode, partition=2)
    assert plan["split_tokens"] == 0 and plan["kernel"] == 3, plan
    ref = r.oracle_decode()
    for kw in (dict(partition=2), dict(partition=1)):
        out, lse = r.decode(**kw)
        r.assert_decode_close(out, lse, ref)


def test_balanced_partitions_with_causal_chunks():
    """Causal multi-token chunks through both balanced partitions: bf16 pages with up to 16 rows
    per KV head (the balanced bf16 kernel), with and without a sliding window; and int8 per-block
    pages with more row groups than half the resident waves, where a forced balanced partition is
    planned over several rounds."""
    r = Run(_wl(2, 128, 16, 4, [300, 5000, 70, 2100, 4], [4, 1, 3, 2, 4], seed=51))
    r.store_prior()
    r.store_new()
    assert pkv.decode_plan(r.w.batch, r.w.num_q_heads, 2, 128, r.w.max_blocks_per_seq, 16, 4, 2,
                           partition=2)["split_tokens"] == 0
    out, lse = r.decode(partition=2)
    r.assert_decode_close(out, lse)
    out, lse = r.decode(partition=2, window=600)
    r.assert_decode_close(out, lse, r.oracle_decode(window=600))
    rng = np.random.default_rng(52)
    ql = rng.integers(1, 17, size=40)
    ctx = ql + rng.integers(0, 700, size=40)
    r = Run(_wl(1, 128, 16, 5, list(ctx), list(ql), hkv=8, seed=53))
    r.store_prior()
    r.store_new()
    plan = pkv.decode_plan(r.w.batch, r.w.num_q_heads, 8, 128, r.w.max_blocks_per_seq, 16, int(ql.max()), 1,
                           partition=2)
    assert plan["split_tokens"] == 0 and plan["num_splits"] > 2048, plan  # several rounds
    out, lse = r.decode(partition=2)
    r.assert_decode_close(out, lse)


def test_planned_partition_matches_fixed_splits():
    """The balanced partition and fixed splits differ only in rounding (fp16 weights against
    different running maxima; bf16 output)."""
    r = Run(_wl(0, 128, 16, 4, [3000, 1200, 4096, 64, 900], seed=15), with_oracle=False)
    r.store_prior()
    r.store_new()
    planned, lp = r.decode(partition=2)
    fixed, lf = r.decode(split_tokens=4096)
    planned2, lp2 = r.decode(partition=2)
    torch.cuda.synchronize()
    assert torch.equal(planned.view(torch.int16), planned2.view(torch.int16))
    diff = (planned.float() - fixed.float()).abs()
    bound = fixed.float().abs() * 2.0 ** -7 + 2.0 ** -10 * float(fixed.float().abs().max())
    assert bool((diff <= bound).all()), float((diff - bound).max())
    assert torch.allclose(lp, lf, rtol=1e-5, atol=1e-5)


def test_workspace_reused_across_shapes_and_kernels():
    """One workspace, filled with NaN bytes to start with, serves calls of different shapes,
    kernels and partitions in turn: no call depends on what an earlier one left there."""
    ws = torch.full((64 << 20,), 0xFF, dtype=torch.uint8, device="cuda")
    cases = [
        (_wl(0, 128, 16, 4, [3000, 1200, 4096, 64, 900], seed=21), dict(split_tokens=256)),
        (_wl(0, 128, 16, 4, [5000, 10, 2600], hkv=4, seed=22), dict(partition=2)),
        (_wl(1, 64, 32, 8, [700, 1500, 33], seed=23), dict(split_tokens=256, kernel=2)),
        (_wl(1, 64, 32, 8, [700, 1500, 33], seed=23), dict(split_tokens=128)),
        (_wl(0, 128, 16, 4, [3000, 1200, 4096, 64, 900], seed=21), dict(partition=2)),
        (_wl(1, 128, 16, 5, [40, 700, 17, 1500], [16, 9, 16, 3], seed=24), dict(split_tokens=128)),
        (_wl(2, 128, 16, 4, [3000, 0, 5000, 64, 900], seed=25), dict(partition=2)),
        (_wl(2, 128, 16, 4, [3000, 0, 5000, 64, 900], seed=25), dict(split_tokens=512)),
    ]
    runs = {}
    for w, kw in cases:
        key = (w.name, w.seed)
        if key not in runs:
            r = Run(w)
            r.store_prior()
            r.store_new()
            runs[key] = r
        r = runs[key]
        for _ in range(2):
            out, lse = r.decode(workspace=ws, **kw)
            r.assert_decode_close(out, lse)


PER_CHANNEL_CASES = [
    # D, BS, G, context lengths, q_lens
    (128, 16, 4, [1, 2, 15, 16, 17, 127, 128, 129, 300, 1000], None),
    (128, 128, 8, [1, 129, 257, 700, 1500], None),
    (64, 16, 4, [37, 100, 5, 260], None),
    (64, 32, 8, [33, 64, 65, 500], None),
    (128, 16, 16, [77, 600], None),
    (128, 16, 5, [20, 40, 16, 300], [3, 16, 1, 7]),
    (128, 64, 2, [300, 31], [12, 31]),
]


@pytest.mark.parametrize("d,bs,g,ctx,ql", PER_CHANNEL_CASES)
def test_per_channel_mode_matches_oracle(d, bs, g, ctx, ql):
    """Static per-channel scales (mode 3): codes bit-exact (the scales are inputs and stay as
    given), attention within the bar for fixed splits and the balanced partition."""
    r = Run(_wl(3, d, bs, g, ctx, ql, seed=d + bs + g + len(ctx)))
    ks0, vs0 = r.cache.k_scale.clone(), r.cache.v_scale.clone()
    r.store_prior()
    r.store_new()
    r.assert_cache_equal()
    assert torch.equal(r.cache.k_scale, ks0) and torch.equal(r.cache.v_scale, vs0)
    ref = r.oracle_decode()
    out, lse = r.decode()
    r.assert_decode_close(out, lse, ref)
    for kw in (dict(split_tokens=128), dict(partition=2)):
        o2, l2 = r.decode(**kw)
        r.assert_decode_close(o2, l2, ref)


def test_per_channel_mode_needs_the_int8_score_kernel():
    r = Run(_wl(3, 128, 16, 4, [40, 100], seed=3), with_oracle=False)
    r.store_prior()
    r.store_new()
    for kernel in (1, 2):
        with pytest.raises(pkv.PkvError) as e:
            r.decode(kernel=kernel)
        assert e.value.status == -2  # PKV_ERR_UNSUPPORTED


def test_per_channel_unwritten_slots_do_not_reach_the_output():
    w = _wl(3, 128, 16, 4, [1, 17, 100, 531], seed=78)
    r = Run(w)
    r.cache.k.fill_(127)
    r.cache.v.fill_(-128)
    r.store_prior()
    r.store_new()
    out, lse = r.decode()
    assert torch.isfinite(out.float()).all()
    r.assert_decode_close(out, lse)


WINDOW_CASES = [
    # mode, D, BS, G, context lengths, q_lens, window
    (0, 128, 16, 4, [1, 17, 300, 1000, 2000], None, 256),
    (0, 128, 128, 8, [129, 700, 1500], None, 100),
    (1, 128, 16, 5, [20, 400, 16, 300], [3, 16, 1, 7], 64),
    (2, 128, 16, 4, [50, 700, 129], None, 200),
    (3, 64, 32, 8, [33, 500, 65], None, 129),
    (0, 64, 16, 2, [300, 31], [12, 31], 1),
]


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("mode,d,bs,g,ctx,ql,window", WINDOW_CASES)
def test_sliding_window_matches_oracle(mode, d, bs, g, ctx, ql, window, kernel):
    """Sliding-window decode (MojoSlidingWindowAttention, Mojo Opset README Op List): each query sees its last `window` positions; the key
    ranges start at the window (128-aligned), so only those blocks are read."""
    if mode == 3 and kernel != 3:
        pytest.skip("the per-channel mode is served by the int8-score kernel only")
    r = Run(_wl(mode, d, bs, g, ctx, ql, seed=sum(ctx) + window))
    r.store_prior()
    r.store_new()
    ref = r.oracle_decode(window=window)
    out, lse = r.decode(kernel=kernel, window=window)
    r.assert_decode_close(out, lse, ref)
    o2, l2 = r.decode(kernel=kernel, window=window, split_tokens=128)
    r.assert_decode_close(o2, l2, ref)
    if kernel == 3:
        o3, l3 = r.decode(kernel=kernel, window=window, partition=2)
        r.assert_decode_close(o3, l3, ref)
    # a window longer than every context is no window at all, bit for bit
    full, lf = r.decode(kernel=kernel)
    big, lb = r.decode(kernel=kernel, window=1 << 30)
    torch.cuda.synchronize()
    assert torch.equal(full.view(torch.int16), big.view(torch.int16)) and torch.equal(lf, lb)
