"""GPU parity of the tile kernel (kernel 4: one workgroup per 128 query rows of a (sequence, KV
head), each 64-key block loaded once per workgroup and shared through LDS) with the oracle.

Cases: whole prompts and chunks after a prior, per-token and per-block scales, tiles partly filled, one and
sixteen query heads per KV head, block-edge lengths, a sequence with no query; key splits (contexts
past 4096 keys with few tiles, forced split sizes, splits that start inside a page) merged by the
log-sum-exp merge; a long prompt in one pass per tile;
softmax scales 0 and negative; query rows with an outlier channel; arguments the kernel does not serve.  Same bars as
test_gpu_parity (attention 1e-2, lse 1e-4 + 1e-5 |lse| + the fp32 evaluation bound)."""
import numpy as np
import pytest
import torch

import gen
import paged_kv_cache_c8_amd as pkv
from tests.gpu_harness import Run
from tests.test_gpu_edge_cases import OUTLIER_CASES, SCALE_CASES, _wl as edge_wl

pytestmark = pytest.mark.gpu

TILE = 4


def _wl(mode, bs, g, ctx, ql, hkv=2, seed=0):
    return gen.custom_workload(f"tile-m{mode}-bs{bs}-g{g}", batch=len(ctx), num_q_heads=hkv * g,
                               num_kv_heads=hkv, head_dim=128, block_size=bs, quant_mode=mode,
                               context_lengths=ctx, q_lens=ql, seed=seed)


TILE_CASES = [
    # mode, BS, G, context lengths, q_lens, KV heads
    (0, 16, 4, [512, 300], [512, 300], 2),              # whole prompts: 16 and 10 tiles of 128 rows
    (1, 16, 5, [1200, 700, 40], [400, 700, 3], 2),       # chunks after a prior; a 15-row tile
    (1, 128, 8, [1000, 129], [600, 129], 1),             # 128-slot pages, eight heads per KV head
    (0, 64, 1, [2000, 65, 1], [2000, 65, 1], 2),         # one query head per KV head
    (1, 32, 6, [100, 1000, 3], [16, 16, 3], 2),          # chunk-sized: one partly filled tile each
    (0, 16, 16, [77, 600, 5], [77, 37, 5], 1),           # sixteen query heads per KV head
    (0, 16, 4, [64, 65, 63, 128, 129], [64, 1, 63, 2, 129], 2),  # lengths at block edges
    (1, 16, 4, [300, 0, 90], [20, 0, 90], 2),            # a sequence with no query and no key
]


@pytest.mark.parametrize("case", TILE_CASES)
def test_tile_kernel_matches_oracle(case):
    mode, bs, g, ctx, ql, hkv = case
    r = Run(_wl(mode, bs, g, ctx, ql, hkv=hkv, seed=sum(ctx) + 7 * mode))
    r.store_prior()
    r.store_new()
    r.assert_cache_equal()
    ref = r.oracle_decode(nthreads=16)
    out, lse = r.decode(kernel=TILE)
    max_abs, rel = r.assert_decode_close(out, lse, ref)
    print(f"  tile mode {mode} bs {bs} g {g}: max_abs={max_abs:.2e} rel={rel:.2e}")


SPLIT_CASES = [
    # mode, BS, G, context lengths, q_lens, KV heads, split_tokens (0: the planner's; these few tiles
    # take splits of 4096 past 4096 keys)
    (1, 16, 5, [5000, 9000, 300, 4097], [16, 9, 3, 1], 2, 0),   # chunk-sized queries on long contexts
    (0, 16, 4, [4500, 70], [300, 70], 1, 0),                     # a prompt chunk over 2 splits
    (0, 16, 4, [9000, 4000], [600, 300], 2, 2048),               # long prompt chunks, 5 splits
    (0, 16, 4, [1200, 700, 40], [400, 700, 3], 2, 64),           # one 64-key block per split
    (1, 16, 5, [1200, 700, 40], [400, 700, 3], 2, 256),
    (1, 16, 6, [3000, 1000, 0], [128, 16, 0], 2, 1024),          # and a sequence with no key
    (1, 128, 8, [1000, 129], [600, 129], 1, 64),                 # splits that start inside a page
    (0, 64, 1, [2000, 65, 1], [2000, 65, 1], 2, 100),            # rounded up to 128 keys
    (1, 32, 4, [6000, 100, 4096], [40, 100, 33], 2, 0),          # 32-slot pages, per-block scales
    (0, 64, 8, [2500, 2600, 17], [16, 2600, 17], 1, 512),        # 64-slot pages, eight heads per KV head
]


@pytest.mark.parametrize("case", SPLIT_CASES)
def test_tile_kernel_key_splits_match_oracle(case):
    mode, bs, g, ctx, ql, hkv, split = case
    r = Run(_wl(mode, bs, g, ctx, ql, hkv=hkv, seed=sum(ctx) + 11 * mode + split))
    r.store_prior()
    r.store_new()
    ref = r.oracle_decode(nthreads=16)
    out, lse = r.decode(kernel=TILE, split_tokens=split)
    max_abs, rel = r.assert_decode_close(out, lse, ref)
    print(f"  tile splits {split or 'auto'} mode {mode} bs {bs} g {g}: max_abs={max_abs:.2e} rel={rel:.2e}")


@pytest.mark.parametrize("case", [c for c in SCALE_CASES if c[0] in (0, 1) and c[1] == 128])
def test_tile_kernel_zero_and_negative_scales(case):
    """Scale 0 (each row's output is the mean of the V rows it sees, lse = log of their count) and
    negative scales (the logits flip), on the inputs the other kernels' scale test uses."""
    mode, d, bs, g, ctx, ql = case
    r = Run(edge_wl(mode, d, bs, g, ctx, ql, seed=97 + mode))
    r.store_prior()
    r.store_new()
    for scale in (0.0, -1.0 / np.sqrt(d), -0.7):
        ref = r.oracle_decode(scale=scale)
        out, lse = r.decode(scale=scale, kernel=TILE)
        r.assert_decode_close(out, lse, ref, scale=scale)


@pytest.mark.parametrize("factor", [64, 256])
@pytest.mark.parametrize("case", [c for c in OUTLIER_CASES if c[0] in (0, 1) and c[1] == 128])
def test_tile_kernel_query_outlier_channels(case, factor):
    """Query rows with one channel 64 or 256 times the rest (exact in bf16), on the inputs the other
    kernels' outlier test uses: the fp16 query is scaled by a power of two relative to the row's
    largest element; the bar must hold anyway."""
    mode, d, bs, g, ctx, ql = case
    w = edge_wl(mode, d, bs, g, ctx, ql, seed=101 + factor + mode)
    t = gen.gen_tensors(w, device=torch.device("cuda"))
    q = t["q"]
    rng = np.random.default_rng(factor + mode)
    ch = torch.as_tensor(rng.integers(0, d, size=q.shape[:2]), device=q.device)
    mult = torch.ones_like(q, dtype=torch.float32)
    mult.scatter_(2, ch.unsqueeze(2), float(factor))
    t["q"] = (q.float() * mult).to(torch.bfloat16)
    assert torch.equal(t["q"].float(), q.float() * mult)
    r = Run(w, tensors=t)
    r.store_prior()
    r.store_new()
    ref = r.oracle_decode()
    o64 = ref[1]
    floor = float(np.abs(o64 - torch.as_tensor(o64).to(torch.bfloat16).double().numpy()).max())
    out, lse = r.decode(kernel=TILE)
    max_abs, rel = r.assert_decode_close(out, lse, ref)
    print(f"  tile outlier x{factor} mode {mode}: max_abs={max_abs:.2e} rel={rel:.2e} "
          f"(bf16 rounding of the oracle itself: {floor:.2e})")


def test_tile_kernel_matches_int8_score_kernel_on_the_prefill_workload():
    """The paged-prefill workload (4 prompts of 2048 tokens, Qwen3-8B heads) on both kernels: every
    element within the attention bar of the other (the oracle is too slow at this size; both sides
    are held to the oracle on the cases above)."""
    w = gen.make_config(5)
    r = Run(w, with_oracle=False)
    r.store_prior()
    r.store_new()
    o3, l3 = r.decode(kernel=3)
    o4, l4 = r.decode(kernel=TILE)
    a, b = o3.float(), o4.float()
    err = (a - b).abs()
    assert torch.all(err <= 2e-2 + 2e-2 * a.abs()), float(err.max())
    assert torch.allclose(l3, l4, rtol=1e-4, atol=1e-3), float((l3 - l4).abs().max())


def test_tile_kernel_unsplit_long_prompt_matches_int8_score_kernel():
    """One prompt of 8192 tokens (2048 tiles, enough to fill the GPU: one pass over up to 8192 keys
    per tile, no key splits, the block-table entries loaded per thread) on both kernels, every
    element within the attention bar of the other."""
    w = gen.make_config(5, prompt_len=8192)
    plan = pkv.decode_plan(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.max_blocks_per_seq,
                           w.block_size, w.max_q_len, w.quant_mode)
    assert plan["kernel"] == TILE and plan["num_splits"] == 1
    r = Run(w, with_oracle=False)
    r.store_prior()
    r.store_new()
    o3, l3 = r.decode(kernel=3)
    o4, l4 = r.decode()
    a, b = o3.float(), o4.float()
    err = (a - b).abs()
    assert torch.all(err <= 2e-2 + 2e-2 * a.abs()), float(err.max())
    assert torch.allclose(l3, l4, rtol=1e-4, atol=1e-3), float((l3 - l4).abs().max())


def test_tile_kernel_rejects_what_it_does_not_serve():
    w64 = gen.custom_workload("tile-d64", batch=1, num_q_heads=8, num_kv_heads=2, head_dim=64, block_size=16,
                              quant_mode=0, context_lengths=[100], q_lens=[100], seed=1)
    r = Run(w64, with_oracle=False)
    with pytest.raises(pkv.PkvError):
        r.decode(kernel=TILE)
    for mode in (2, 3):  # bf16 pages; static per-channel scales (the int8-score kernel's)
        r = Run(_wl(mode, 16, 4, [100], [100], seed=2), with_oracle=False)
        with pytest.raises(pkv.PkvError):
            r.decode(kernel=TILE)
    w = _wl(0, 16, 4, [300], [300], seed=3)
    r = Run(w, with_oracle=False)
    for kw in (dict(window=128), dict(partition=1)):
        with pytest.raises(pkv.PkvError):
            r.decode(kernel=TILE, **kw)
