"""The debug validator (pkv_check_indices) on the GPU: it passes every index array a valid workload
holds, flags each kind of out-of-range entry (context lengths, block-table entries the context
reaches, query-length prefix sums, slot mapping) with the lowest offending sequence or token, and
ignores entries no call reads (block-table entries past the context, negative slots).  Under
PKV_CHECK=1 the binding runs it first and raises PkvIndexError instead of making a store, dequant or
decode call with such arrays; those calls then launch nothing that reads them."""
import numpy as np
import pytest
import torch

import gen
import paged_kv_cache_c8_amd as pkv
from tests.gpu_harness import Run

pytestmark = pytest.mark.gpu


def _run():
    w = gen.custom_workload("check", batch=4, num_q_heads=8, num_kv_heads=2, head_dim=64, block_size=16,
                            quant_mode=0, context_lengths=[1, 40, 0, 100], q_lens=[1, 5, 0, 3], seed=7,
                            max_blocks_per_seq=9)
    return Run(w, with_oracle=False)


def test_valid_workload_passes():
    r = _run()
    assert pkv.check_indices(r.cache, r.bt, r.ctx, cu_q_lens=r.cu_q, max_q_len=5) == (0, -1, -1)
    slots = torch.tensor([0, 17, -1, r.cache.num_blocks * 16 - 1], dtype=torch.int64, device="cuda")
    assert pkv.check_indices(r.cache, slot_mapping=slots) == (0, -1, -1)


def test_each_violation_is_flagged_with_its_first_index():
    r = _run()
    nb = r.cache.num_blocks
    bt = r.bt.clone()
    bt[3, 5] = nb  # sequence 3 (100 keys, 7 pages) reaches entry 5
    assert pkv.check_indices(r.cache, bt, r.ctx) == (pkv.CHECK_BLOCK, 3, -1)
    bt[1, 2] = -3  # sequence 1 (40 keys) reaches entries 0..2
    assert pkv.check_indices(r.cache, bt, r.ctx) == (pkv.CHECK_BLOCK, 1, -1)
    past = r.bt.clone()
    past[1, 3] = 10 ** 6  # past sequence 1's context: never read, not flagged
    past[2, 0] = -1  # sequence 2 is empty
    assert pkv.check_indices(r.cache, past, r.ctx) == (0, -1, -1)
    ctx = r.ctx.clone()
    ctx[2] = -1
    assert pkv.check_indices(r.cache, r.bt, ctx) == (pkv.CHECK_CONTEXT, 2, -1)
    ctx[2] = 9 * 16 + 1  # more keys than the table's row holds
    flags, seq, _ = pkv.check_indices(r.cache, r.bt, ctx)
    assert flags & pkv.CHECK_CONTEXT and seq == 2
    cu = r.cu_q.clone()
    cu[2] = cu[1] - 1  # decreasing
    assert pkv.check_indices(r.cache, r.bt, r.ctx, cu_q_lens=cu)[0] == pkv.CHECK_QLEN
    assert pkv.check_indices(r.cache, r.bt, r.ctx, cu_q_lens=r.cu_q, max_q_len=4) == (pkv.CHECK_QLEN, 1, -1)
    cu = r.cu_q.clone()
    cu[1:] += 1  # sequence 0: 2 new tokens for a context of 1
    assert pkv.check_indices(r.cache, r.bt, r.ctx, cu_q_lens=cu)[:2] == (pkv.CHECK_QLEN, 0)
    slots = torch.tensor([3, -5, nb * 16, 2, nb * 16 + 7], dtype=torch.int64, device="cuda")
    assert pkv.check_indices(r.cache, slot_mapping=slots) == (pkv.CHECK_SLOT, -1, 2)


def test_large_table_is_checked_whole():
    """More entries than the check's workgroup has threads: the offending entry is the last one."""
    batch, mbs, nb = 300, 64, 300 * 64
    ctx = torch.full((batch,), mbs * 16, dtype=torch.int32, device="cuda")
    bt = torch.arange(batch * mbs, dtype=torch.int32, device="cuda").reshape(batch, mbs)
    cache = pkv.Cache(0, nb, 1, 16, 64)
    assert pkv.check_indices(cache, bt, ctx) == (0, -1, -1)
    bt[batch - 1, mbs - 1] = nb
    assert pkv.check_indices(cache, bt, ctx) == (pkv.CHECK_BLOCK, batch - 1, -1)


def test_pkv_check_stops_calls_with_bad_indices(monkeypatch):
    r = _run()
    r.store_prior()
    r.store_new()
    bt = r.bt.clone()
    bt[3, 6] = r.cache.num_blocks + 100  # in sequence 3's context: would be read
    q = r.queries()
    monkeypatch.setenv("PKV_CHECK", "1")
    out = torch.full_like(q, 3.0)
    with pytest.raises(pkv.PkvIndexError, match="block-table entry"):
        pkv.decode_gqa(q, r.cache, bt, r.ctx, 0.125, cu_q_lens=r.cu_q, max_q_len=5, out=out)
    with pytest.raises(pkv.PkvIndexError):
        pkv.decode_gqa_noalloc(q, r.cache, bt, r.ctx, 0.125, out, cu_q_lens=r.cu_q, max_q_len=5)
    with pytest.raises(pkv.PkvIndexError):
        pkv.dequant(r.cache, bt, r.ctx, num_rows=141)
    with pytest.raises(pkv.PkvIndexError, match="query lengths"):
        pkv.decode_gqa(q, r.cache, r.bt, r.ctx, 0.125, cu_q_lens=r.cu_q, max_q_len=2, out=out)
    kn = torch.zeros((2, 2, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(pkv.PkvIndexError, match="slot mapping"):
        pkv.store_c8(r.cache, kn, kn, slot_mapping=torch.tensor([0, 10 ** 9], dtype=torch.int64, device="cuda"))
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())  # nothing was launched into out
    # valid arrays pass through the check and give the result of the unchecked call
    got = pkv.decode_gqa(q, r.cache, r.bt, r.ctx, 0.125, cu_q_lens=r.cu_q, max_q_len=5)
    monkeypatch.delenv("PKV_CHECK")
    want = pkv.decode_gqa(q, r.cache, r.bt, r.ctx, 0.125, cu_q_lens=r.cu_q, max_q_len=5)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), want.view(torch.int16))


def test_mla_calls_are_checked(monkeypatch):
    cache = pkv.MLACache(8, 16)
    ctx = torch.tensor([20, 5], dtype=torch.int32, device="cuda")
    bt = torch.tensor([[0, 9], [1, 2]], dtype=torch.int32, device="cuda")  # entry 9 of an 8-block pool
    assert pkv.check_indices(cache, bt, ctx) == (pkv.CHECK_BLOCK, 0, -1)
    monkeypatch.setenv("PKV_CHECK", "1")
    q = torch.zeros((2, 16, 512), dtype=torch.bfloat16, device="cuda")
    qr = torch.zeros((2, 16, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(pkv.PkvIndexError):
        pkv.mla_decode(q, qr, cache, bt, ctx, 0.1)
