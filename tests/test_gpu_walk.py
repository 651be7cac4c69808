"""pkv_cache_walk (the read-ceiling walker): every wave's checksum equals the wrapping sum of the
32-bit words of exactly the cache bytes the decode of its keys reads - K rows of its keys, whole
16-slot V tiles that hold them, per-token scales of its keys or the per-block scales of the pages
it touches (once per wave) - recomputed on the host from the cache's bytes.  A wrong page, slot,
tile, lane mapping or a read past the context changes a sum."""
import numpy as np
import pytest
import torch

import gen
import paged_kv_cache_c8_amd as pkv
from tests.gpu_harness import Run

pytestmark = pytest.mark.gpu


def expected_sums(cache, w, split):
    k = cache.k.view(torch.uint8).cpu().numpy()
    v = cache.v.view(torch.uint8).cpu().numpy().reshape(w.num_blocks, w.num_kv_heads, w.block_size // 16, -1)
    ks = cache.k_scale.cpu().numpy().view(np.uint32) if cache.k_scale is not None else None
    vs = cache.v_scale.cpu().numpy().view(np.uint32) if cache.v_scale is not None else None
    bs = w.block_size
    nsplit = -(-w.max_blocks_per_seq * bs // split)
    out = np.zeros((w.batch, w.num_kv_heads, nsplit), dtype=np.uint64)
    for b in range(w.batch):
        ctx = int(w.context_lengths[b])
        for h in range(w.num_kv_heads):
            for s in range(nsplit):
                t0, t1 = s * split, min((s + 1) * split, ctx)
                if t0 >= t1:
                    continue
                tot = 0
                for p in range(t0, t1):
                    page, slot = int(w.block_table[b, p // bs]), p % bs
                    tot += int(k[page, h, slot].view(np.uint32).sum(dtype=np.uint64))
                    if w.quant_mode == 0:
                        tot += int(ks[page, h, slot]) + int(vs[page, h, slot])
                for tg in range(t0, t1, 16):
                    page, tile = int(w.block_table[b, tg // bs]), (tg % bs) // 16
                    tot += int(v[page, h, tile].view(np.uint32).sum(dtype=np.uint64))
                if w.quant_mode == 1:
                    for j in range(t0 // bs, (t1 - 1) // bs + 1):
                        page = int(w.block_table[b, j])
                        tot += int(ks[page, h]) + int(vs[page, h])
                out[b, h, s] = tot & 0xffffffff
    return out.astype(np.uint32)


@pytest.mark.parametrize("mode,d,bs,ctx,split", [
    (0, 128, 16, [0, 1, 63, 64, 65, 1000, 3000], 384),
    (0, 64, 32, [17, 129, 700], 64),
    (1, 128, 128, [1, 200, 1000], 64),     # splits start inside pages (each page once per wave)
    (1, 64, 16, [130, 5, 64], 128),
    (3, 128, 32, [300, 0, 2049], 256),
])
def test_walk_checksums(mode, d, bs, ctx, split):
    w = gen.custom_workload(f"walk-m{mode}", batch=len(ctx), num_q_heads=8, num_kv_heads=2, head_dim=d,
                            block_size=bs, quant_mode=mode, context_lengths=ctx, seed=sum(ctx) + bs)
    r = Run(w, with_oracle=False, fill=0x35)  # unwritten slots hold a nonzero byte
    r.store_prior()
    r.store_new()
    want = expected_sums(r.cache, w, split)
    for depth in (1, 2, 3):
        got = pkv.cache_walk(r.cache, r.bt, r.ctx, split, depth=depth)
        torch.cuda.synchronize()
        got = got.cpu().numpy().view(np.uint32)
        assert np.array_equal(got, want), (depth, np.argwhere(got != want)[:5].tolist())


def test_walk_rejects_bf16_and_bad_splits():
    w = gen.custom_workload("walk-bad", batch=2, num_q_heads=4, num_kv_heads=1, head_dim=64, block_size=16,
                            quant_mode=2, context_lengths=[5, 9], seed=1)
    r = Run(w, with_oracle=False)
    with pytest.raises(pkv.PkvError):
        pkv.cache_walk(r.cache, r.bt, r.ctx, 64)
    w = gen.custom_workload("walk-bad2", batch=2, num_q_heads=4, num_kv_heads=1, head_dim=64, block_size=16,
                            quant_mode=0, context_lengths=[5, 9], seed=1)
    r = Run(w, with_oracle=False)
    for split, depth in ((96, 1), (0, 1), (8192, 1), (64, 4), (64, 0)):
        with pytest.raises(pkv.PkvError):
            pkv.cache_walk(r.cache, r.bt, r.ctx, split, depth=depth)


def mla_expected_sums(cache, w, split):
    """Per (sequence, split): the wrapping sum of the 32-bit words of the latent row, the rotary row
    and the two scales of every key in the split's range, from the cache's bytes."""
    lat = cache.latent.view(torch.uint8).cpu().numpy().reshape(w.num_blocks * w.block_size, -1)
    rope = cache.rope.view(torch.uint8).cpu().numpy().reshape(w.num_blocks * w.block_size, -1)
    ls = cache.latent_scale.cpu().numpy().reshape(-1).view(np.uint32).astype(np.uint64)
    rs = cache.rope_scale.cpu().numpy().reshape(-1).view(np.uint32).astype(np.uint64)
    row_words = (np.ascontiguousarray(lat).view(np.uint32).sum(axis=1, dtype=np.uint64)
                 + np.ascontiguousarray(rope).view(np.uint32).sum(axis=1, dtype=np.uint64) + ls + rs)
    bs = w.block_size
    nsplit = -(-w.max_blocks_per_seq * bs // split)
    out = np.zeros((w.batch, nsplit), dtype=np.uint64)
    for b in range(w.batch):
        ctx = int(w.context_lengths[b])
        pos = np.arange(ctx)
        rows = w.block_table[b, pos // bs].astype(np.int64) * bs + pos % bs
        for s in range(nsplit):
            t0, t1 = s * split, min((s + 1) * split, ctx)
            if t0 < t1:
                out[b, s] = int(row_words[rows[t0:t1]].sum(dtype=np.uint64)) & 0xffffffff
    return out.astype(np.uint32)


@pytest.mark.parametrize("bs,ctx,split", [
    (16, [0, 1, 63, 64, 65, 1000, 3000], 64),
    (64, [37, 2048, 4095, 130], 640),
    (128, [1, 700, 8192], 4096),
    (32, [200, 17], 192),   # splits start inside pages
])
def test_mla_walk_checksums(bs, ctx, split):
    from tests.test_gpu_mla import MlaRun

    w = gen.mla_workload(f"mla-walk-{bs}", batch=len(ctx), num_heads=16, block_size=bs, context_lengths=ctx,
                         seed=sum(ctx) + bs)
    r = MlaRun(w)
    # unwritten rows hold nonzero bytes and scales, so a read past a context changes a sum
    r.cache.latent.fill_(53)
    r.cache.rope.fill_(-7)
    r.cache.latent_scale.fill_(0.25)
    r.cache.rope_scale.fill_(3.0)
    r.store()
    want = mla_expected_sums(r.cache, w, split)
    got = pkv.mla_cache_walk(r.cache, r.bt, r.ctx, split)
    torch.cuda.synchronize()
    got = got.cpu().numpy().view(np.uint32)
    assert np.array_equal(got, want), np.argwhere(got != want)[:5].tolist()
