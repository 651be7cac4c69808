"""pkv_store_decode_gqa (one decode step: store each sequence's new token, then attend) against the
two calls it stands for, pkv_store_c8 then pkv_decode_gqa, and against the oracle.

Where the store is fused into the int8-score decode (per-token and per-channel caches, one row
group per KV head) the wave that attends to the new position quantizes the token, writes it and
uses its codes from LDS; elsewhere a store launch precedes the decode.  Either way the cache bytes,
the outputs and the lse must be bit for bit those of the two calls (the same quantization and the
same plan), and within the bar of the oracle."""
import numpy as np
import pytest
import torch

import gen
import oracle
import paged_kv_cache_c8_amd as pkv
from tests.gpu_harness import Run, bits

pytestmark = pytest.mark.gpu

CASES = [
    # mode, D, BS, G, context lengths (0: an empty slot), options
    (0, 128, 16, 4, [1, 2, 64, 65, 128, 129, 1000, 3000], {}),                    # fused, fixed splits
    (0, 128, 16, 4, [1, 2, 64, 65, 128, 129, 1000, 3000], dict(split_tokens=128)),
    (0, 128, 128, 8, [20000, 129, 40000, 1], dict(partition=2)),                  # fused, balanced
    (0, 128, 16, 4, [0, 77, 0, 300], {}),                                         # empty sequences
    (3, 128, 16, 4, [17, 500, 2049], {}),                                         # per channel, fused
    (3, 64, 32, 8, [33, 4097, 65], dict(partition=2)),
    (0, 64, 16, 16, [300, 1, 129], {}),                                           # 16 rows, fused
    (0, 128, 16, 32, [300, 129], {}),                                             # two row groups: store launch
    (1, 128, 16, 4, [20, 129, 300], {}),                                          # per block: store launch
    (2, 128, 16, 4, [1, 300, 5000], {}),                                          # bf16: store launch
    (0, 128, 16, 4, [1, 300, 1000], dict(kernel=1)),                              # VALU kernel: store launch
    (0, 128, 16, 4, [90, 3000], dict(window=100)),                                # sliding window, fused
]


@pytest.mark.parametrize("mode,d,bs,g,ctx,kw", CASES)
def test_store_decode_equals_store_then_decode(mode, d, bs, g, ctx, kw):
    w = gen.custom_workload(f"store-decode-m{mode}", batch=len(ctx), num_q_heads=2 * g, num_kv_heads=2, head_dim=d,
                            block_size=bs, quant_mode=mode, context_lengths=ctx, seed=sum(ctx) + d + g)
    fused = Run(w)
    two = Run(w, tensors=fused.t)
    for r in (fused, two):
        r.store_prior()
    scale = 1.0 / np.sqrt(d)
    q = fused.queries()
    kn, vn = fused._decode_rows(fused.k_new), fused._decode_rows(fused.v_new)
    lse_f = torch.full((w.batch, w.num_q_heads), 7.0, dtype=torch.float32, device=q.device)
    out_f = pkv.store_decode_gqa(q, kn, vn, fused.cache, fused.bt, fused.ctx, scale, lse_out=lse_f, **kw)
    two.store_new()
    out_t, lse_t = two.decode(**kw)
    torch.cuda.synchronize()
    for name in ("k", "v", "k_scale", "v_scale"):
        a, b = getattr(fused.cache, name), getattr(two.cache, name)
        if a is not None:
            assert torch.equal(a.view(torch.uint8) if a.dtype != torch.float32 else a.view(torch.int32),
                               b.view(torch.uint8) if b.dtype != torch.float32 else b.view(torch.int32)), name
    assert torch.equal(out_f.view(torch.int16), out_t.view(torch.int16))
    assert torch.equal(lse_f, lse_t)
    # the oracle's cache takes the same new tokens (the harness's store_new was not used for `fused`)
    oracle.store(fused.hc, bits(kn), bits(vn), context_lengths=w.context_lengths, block_table=w.block_table)
    fused.assert_cache_equal()
    window = kw.get("window", 0)
    fused.assert_decode_close(out_f, lse_f, fused.oracle_decode(window=window), scale=scale)


def test_store_decode_repeated_steps():
    """Several decode steps in a row, each storing one more token per sequence (the new token of
    one step is an ordinary cached key of the next), against the two-call path."""
    ctx0 = np.array([100, 1023, 4000, 1])
    steps = 5
    w = gen.custom_workload("store-decode-steps", batch=4, num_q_heads=8, num_kv_heads=2, head_dim=128,
                            block_size=16, quant_mode=0, context_lengths=list(ctx0 + steps - 1), seed=3)
    dev = torch.device("cuda")
    t = gen.gen_tensors(w, device=dev)
    bt = torch.as_tensor(w.block_table, device=dev)
    caches = [pkv.Cache(0, w.num_blocks, 2, 16, 128, device=dev) for _ in range(2)]
    cu = w.cu_context
    # the tokens before the first step, in one prompt-style store
    rows = torch.as_tensor(np.concatenate([np.arange(cu[b], cu[b] + ctx0[b] - 1) for b in range(4)]), device=dev)
    cu_p = torch.as_tensor(np.concatenate([[0], np.cumsum(ctx0 - 1)]).astype(np.int32), device=dev)
    for c in caches:
        pkv.store_c8(c, t["k_all"].index_select(0, rows), t["v_all"].index_select(0, rows), cu_q_lens=cu_p,
                     context_lengths=torch.as_tensor((ctx0 - 1).astype(np.int32), device=dev), block_table=bt,
                     max_q_len=int(ctx0.max()))
    gq = torch.Generator(device=dev).manual_seed(9)
    for step in range(steps):
        ctx = torch.as_tensor((ctx0 + step).astype(np.int32), device=dev)
        new = torch.as_tensor(np.array([cu[b] + ctx0[b] - 1 + step for b in range(4)]), device=dev)
        kn, vn = t["k_all"].index_select(0, new).contiguous(), t["v_all"].index_select(0, new).contiguous()
        q = torch.randn((4, 8, 128), generator=gq, device=dev).to(torch.bfloat16)
        out_f = pkv.store_decode_gqa(q, kn, vn, caches[0], bt, ctx, 0.1)
        pkv.store_c8(caches[1], kn, vn, context_lengths=ctx, block_table=bt)
        out_t = pkv.decode_gqa(q, caches[1], bt, ctx, 0.1)
        torch.cuda.synchronize()
        assert torch.equal(out_f.view(torch.int16), out_t.view(torch.int16)), step
        assert torch.equal(caches[0].k, caches[1].k) and torch.equal(caches[0].v, caches[1].v)
        assert torch.equal(caches[0].k_scale, caches[1].k_scale) and torch.equal(caches[0].v_scale, caches[1].v_scale)
