"""The calls under HIP graph capture (torch.cuda.CUDAGraph).  The library's work is plain kernel
launches on the caller's stream (no memset, no allocation, no host synchronisation), so a capture
records them as they are.  Each captured call is replayed several times with new inputs written
between the replays (eager work, then a synchronisation), and every replay must equal, bit for
bit, the same call made eagerly: the decode (fixed splits, the balanced partition, causal chunks,
bf16 pages), the decode with no workspace (the entry point for callers that cannot allocate), and
the one-call decode steps (GQA and MLA) whose store rewrites the cache on every replay."""
import numpy as np
import pytest
import torch

import gen
import paged_kv_cache_c8_amd as pkv
from tests.gpu_harness import Run

pytestmark = pytest.mark.gpu

REPLAYS = 4

CASES = [
    # name, mode, D, BS, G, context lengths, q lens (None: one query each), call options
    ("fixed", 0, 128, 16, 4, [1, 300, 1025, 4000], None, {}),
    ("balanced", 0, 128, 128, 8, [20000, 129, 40000], None, dict(partition=2)),
    ("per-channel", 3, 128, 16, 4, [17, 2049, 700], None, {}),
    ("chunked", 1, 128, 16, 5, [40, 2000, 16], [16, 7, 3], {}),
    ("bf16", 2, 128, 16, 4, [64, 5000, 300], None, {}),
]


def _bf16(shape, gen_):
    return torch.randn(shape, generator=gen_, device="cuda").to(torch.bfloat16)


@pytest.mark.parametrize("name,mode,d,bs,g,ctx,ql,kw", CASES, ids=[c[0] for c in CASES])
def test_captured_decode_replays_equal_eager(name, mode, d, bs, g, ctx, ql, kw):
    w = gen.custom_workload(f"graph-{name}", batch=len(ctx), num_q_heads=2 * g, num_kv_heads=2, head_dim=d,
                            block_size=bs, quant_mode=mode, context_lengths=ctx, q_lens=ql, seed=sum(ctx) + d)
    r = Run(w, with_oracle=False)
    r.store_prior()
    r.store_new()
    q0 = r.queries()
    hq = w.num_q_heads
    need = pkv.decode_workspace_size(w.batch, hq, r.cache, w.max_blocks_per_seq, w.max_q_len, **kw)
    ws_g = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    ws_e = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    q_in = q0.clone()
    out_g = torch.empty_like(q0)
    lse_g = torch.empty((q0.shape[0], hq), dtype=torch.float32, device="cuda")
    call = lambda q, out, lse, ws: pkv.decode_gqa(q, r.cache, r.bt, r.ctx, 0.09, cu_q_lens=r.cu_q,
                                                  max_q_len=w.max_q_len, out=out, lse_out=lse, workspace=ws, **kw)
    call(q_in, out_g, lse_g, ws_g)  # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(q_in, out_g, lse_g, ws_g)
    gq = torch.Generator(device="cuda").manual_seed(21)
    for i in range(REPLAYS):
        qi = _bf16(q0.shape, gq)
        q_in.copy_(qi)
        graph.replay()
        out_e = torch.empty_like(q0)
        lse_e = torch.empty_like(lse_g)
        call(qi, out_e, lse_e, ws_e)
        torch.cuda.synchronize()
        assert torch.equal(out_g.view(torch.int16), out_e.view(torch.int16)), (name, i)
        assert torch.equal(lse_g.view(torch.int32), lse_e.view(torch.int32)), (name, i)


def test_captured_noalloc_decode_replays_equal_eager():
    w = gen.custom_workload("graph-noalloc", batch=4, num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=16,
                            quant_mode=0, context_lengths=[1, 300, 1025, 4000], seed=5)
    r = Run(w, with_oracle=False)
    r.store_prior()
    r.store_new()
    q0 = r.queries()
    q_in, out_g = q0.clone(), torch.empty_like(q0)
    lse_g = torch.empty((4, 8), dtype=torch.float32, device="cuda")
    call = lambda q, out, lse: pkv.decode_gqa_noalloc(q, r.cache, r.bt, r.ctx, 0.09, out, lse_out=lse)
    call(q_in, out_g, lse_g)  # warm-up: takes the scratch array's address outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(q_in, out_g, lse_g)
    gq = torch.Generator(device="cuda").manual_seed(22)
    for i in range(REPLAYS):
        qi = _bf16(q0.shape, gq)
        q_in.copy_(qi)
        graph.replay()
        torch.cuda.synchronize()
        got_o, got_l = out_g.clone(), lse_g.clone()
        out_e, lse_e = torch.empty_like(q0), torch.empty_like(lse_g)
        pkv.decode_gqa(qi, r.cache, r.bt, r.ctx, 0.09, out=out_e, lse_out=lse_e)
        torch.cuda.synchronize()
        assert torch.equal(got_o.view(torch.int16), out_e.view(torch.int16)), i
        assert torch.equal(got_l.view(torch.int32), lse_e.view(torch.int32)), i


@pytest.mark.parametrize("mode", [0, 3, 1])
def test_captured_decode_step_replays_equal_eager(mode):
    """The one-call decode step (store inside the int8 decode for modes 0 and 3; a store launch
    before it for mode 1), captured once and replayed with new tokens and queries: the cache and
    the outputs after every replay equal those of the same step made eagerly on a second cache."""
    ctx = [1, 300, 1025, 4000]
    w = gen.custom_workload(f"graph-step-m{mode}", batch=4, num_q_heads=8, num_kv_heads=2, head_dim=128,
                            block_size=16, quant_mode=mode, context_lengths=ctx, seed=6 + mode)
    ra = Run(w, with_oracle=False)
    rb = Run(w, with_oracle=False, tensors=ra.t)
    for r in (ra, rb):
        r.store_prior()
    shape_q, shape_kv = (4, 8, 128), (4, 2, 128)
    q_in = torch.zeros(shape_q, dtype=torch.bfloat16, device="cuda")
    k_in = torch.zeros(shape_kv, dtype=torch.bfloat16, device="cuda")
    v_in = torch.zeros(shape_kv, dtype=torch.bfloat16, device="cuda")
    out_g = torch.empty(shape_q, dtype=torch.bfloat16, device="cuda")
    need = pkv.decode_workspace_size(4, 8, ra.cache, w.max_blocks_per_seq)
    ws_g = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    step = lambda r, q, k, v, out, ws: pkv.store_decode_gqa(q, k, v, r.cache, r.bt, r.ctx, 0.09, out=out,
                                                            workspace=ws)
    step(ra, q_in, k_in, v_in, out_g, ws_g)  # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(ra, q_in, k_in, v_in, out_g, ws_g)
    gq = torch.Generator(device="cuda").manual_seed(23)
    for i in range(REPLAYS):
        qi, ki, vi = _bf16(shape_q, gq), _bf16(shape_kv, gq), _bf16(shape_kv, gq)
        q_in.copy_(qi)
        k_in.copy_(ki)
        v_in.copy_(vi)
        graph.replay()
        out_e = step(rb, qi, ki, vi, torch.empty_like(out_g), torch.empty_like(ws_g))
        torch.cuda.synchronize()
        assert torch.equal(out_g.view(torch.int16), out_e.view(torch.int16)), (mode, i)
        for name in ("k", "v", "k_scale", "v_scale"):
            a, b = getattr(ra.cache, name), getattr(rb.cache, name)
            if a is not None:
                assert torch.equal(a.view(torch.uint8) if a.dtype != torch.float32 else a.view(torch.int32),
                                   b.view(torch.uint8) if b.dtype != torch.float32 else b.view(torch.int32)), (mode, i, name)


def test_captured_mla_decode_step_replays_equal_eager():
    """The MLA decode step (its store inside the decode launch), captured and replayed with new
    tokens and queries, against the same step made eagerly on a second cache."""
    w = gen.mla_workload("graph-mla", batch=4, num_heads=16, block_size=64, context_lengths=[1, 300, 1025, 4000],
                         seed=8, softmax_scale=0.07)
    t = gen.gen_mla_tensors(w, device="cuda")
    bt = torch.as_tensor(w.block_table, device="cuda")
    ctx = torch.as_tensor(w.context_lengths, device="cuda")
    caches = [pkv.MLACache(w.num_blocks, w.block_size) for _ in range(2)]
    prior = w.prior_lengths
    cu = w.cu_context
    rows = torch.as_tensor(np.concatenate([np.arange(cu[b], cu[b] + prior[b]) for b in range(w.batch)]), device="cuda")
    cu_p = torch.as_tensor(np.concatenate([[0], np.cumsum(prior)]).astype(np.int32), device="cuda")
    for c in caches:
        pkv.mla_store_c8(c, t["latent_all"].index_select(0, rows), t["rope_all"].index_select(0, rows), cu_q_lens=cu_p,
                         context_lengths=torch.as_tensor(prior.astype(np.int32), device="cuda"), block_table=bt)
    shapes = [(4, 16, 512), (4, 16, 64), (4, 512), (4, 64)]
    ins = [torch.zeros(s, dtype=torch.bfloat16, device="cuda") for s in shapes]
    out_g = torch.empty(shapes[0], dtype=torch.bfloat16, device="cuda")
    need = pkv.mla_decode_workspace_size(4, 16, w.max_blocks_per_seq, w.block_size)
    ws_g = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    step = lambda c, x, out, ws: pkv.mla_store_decode(x[0], x[1], x[2], x[3], c, bt, ctx, 0.07, out=out, workspace=ws)
    step(caches[0], ins, out_g, ws_g)  # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(caches[0], ins, out_g, ws_g)
    gq = torch.Generator(device="cuda").manual_seed(24)
    for i in range(REPLAYS):
        xs = [_bf16(s, gq) for s in shapes]
        for dst, src in zip(ins, xs):
            dst.copy_(src)
        graph.replay()
        out_e = step(caches[1], xs, torch.empty_like(out_g), torch.empty_like(ws_g))
        torch.cuda.synchronize()
        assert torch.equal(out_g.view(torch.int16), out_e.view(torch.int16)), i
        for name in ("latent", "rope", "latent_scale", "rope_scale"):
            assert torch.equal(getattr(caches[0], name).view(torch.uint8), getattr(caches[1], name).view(torch.uint8)), (i, name)
