"""pkv_decode_gqa_noalloc (scratch space in a fixed per-GPU array of the library) against
pkv_decode_gqa (caller workspace): the same plan and kernels, so the outputs must agree bit for bit,
and both within the attention bar of the oracle.  Two calls in a row, the second with a smaller
input (the array keeps the first call's partials: the second must not depend on them); a call
whose plan needs more than the array holds is refused before anything runs."""
import numpy as np
import pytest
import torch

import gen
import paged_kv_cache_c8_amd as pkv
from tests.gpu_harness import Run

pytestmark = pytest.mark.gpu


def _wl(mode, ctx, g=4, hkv=8, bs=16, seed=0):
    return gen.custom_workload(f"noalloc-m{mode}", batch=len(ctx), num_q_heads=hkv * g, num_kv_heads=hkv,
                               head_dim=128, block_size=bs, quant_mode=mode, context_lengths=ctx, seed=seed)


def _both(r, **kw):
    w = r.w
    scale = 1.0 / np.sqrt(w.head_dim)
    q = r.queries()
    out_a = torch.full_like(q, float("nan"))
    lse_a = torch.full((q.shape[0], w.num_q_heads), 7.0, dtype=torch.float32, device=q.device)
    pkv.decode_gqa_noalloc(q, r.cache, r.bt, r.ctx, scale, out_a, lse_out=lse_a, **kw)
    out_b, lse_b = r.decode(**kw)
    torch.cuda.synchronize()
    return out_a, lse_a, out_b, lse_b


@pytest.mark.parametrize("kw", [dict(), dict(partition=2), dict(split_tokens=256)])
def test_noalloc_matches_workspace_entry_point(kw):
    rng = np.random.default_rng(7)
    big = Run(_wl(0, list(rng.integers(1024, 4097, size=24)), seed=71))   # fixed splits by default
    small = Run(_wl(0, [700, 1, 33], seed=72))
    for r in (big, small):
        r.store_prior()
        r.store_new()
    assert pkv.decode_workspace_size(big.w.batch, 32, big.cache, big.w.max_blocks_per_seq, **kw) > \
        pkv.decode_workspace_size(small.w.batch, 32, small.cache, small.w.max_blocks_per_seq, **kw)
    for r in (big, small):  # the second call is smaller: what the first left in the array is stale
        out_a, lse_a, out_b, lse_b = _both(r, **kw)
        assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16))
        assert torch.equal(lse_a, lse_b)
        r.assert_decode_close(out_a, lse_a)


def test_noalloc_long_context_balanced_partition():
    """A long-context batch (balanced partition, segment records in the array), then a short one."""
    r1 = Run(_wl(0, [20000, 3000, 40000], g=8, hkv=8, bs=128, seed=73))
    r2 = Run(_wl(1, [300, 17], g=5, hkv=8, seed=74))
    for r in (r1, r2):
        r.store_prior()
        r.store_new()
        out_a, lse_a, out_b, lse_b = _both(r)
        assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16))
        assert torch.equal(lse_a, lse_b)
        r.assert_decode_close(out_a, lse_a)


def test_noalloc_refuses_plans_beyond_its_array():
    """A plan needing more than NOALLOC_SCRATCH_BYTES is refused on the host (PKV_ERR_WORKSPACE),
    nothing launched: the output keeps its contents."""
    w = gen.custom_workload("noalloc-big", batch=64, num_q_heads=40, num_kv_heads=8, head_dim=128, block_size=16,
                            quant_mode=1, context_lengths=[4000] * 64, q_lens=[16] * 64, seed=75)
    cache = pkv.Cache(1, w.num_blocks, 8, 16, 128, device="cuda")
    need = pkv.decode_workspace_size(w.batch, 40, cache, w.max_blocks_per_seq, 16, partition=1)
    assert need > pkv.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((w.num_new_tokens, 40, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.full_like(q, 3.0)
    bt = torch.as_tensor(w.block_table, device="cuda")
    ctx = torch.as_tensor(w.context_lengths, device="cuda")
    cu = torch.as_tensor(w.cu_q_lens, device="cuda")
    with pytest.raises(pkv.PkvError) as e:
        pkv.decode_gqa_noalloc(q, cache, bt, ctx, 0.1, out, cu_q_lens=cu, max_q_len=16, partition=1)
    assert e.value.status == -3
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())
