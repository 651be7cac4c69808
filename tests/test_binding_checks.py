"""Host-side argument checks of the Python binding (no GPU needed).

The kernels trust the sizes they are given, so the binding checks every tensor argument's dtype,
shape, contiguity and device before anything reaches the library.  Here ``lib()`` is replaced by a
function that fails the test if it is called: each bad argument must raise ``ValueError`` first,
and arguments that are right in every respect but live in host memory must be refused as well.
"""
import numpy as np
import pytest
import torch

import paged_kv_cache_c8_amd as pkv


@pytest.fixture(autouse=True)
def no_library(monkeypatch):
    def boom():
        raise AssertionError("the library was called: an argument check is missing")

    monkeypatch.setattr(pkv, "lib", boom)


B, HQ, HKV, D, BS, NB, MBS = 3, 8, 2, 128, 16, 12, 4


def cache(mode=0):
    return pkv.Cache(mode, NB, HKV, BS, D, device="cpu")


def good_decode_args():
    return dict(q=torch.zeros(B, HQ, D, dtype=torch.bfloat16), block_table=torch.zeros(B, MBS, dtype=torch.int32),
                context_lengths=torch.ones(B, dtype=torch.int32), scale=0.1)


def call_decode(c, **over):
    a = good_decode_args()
    a.update(over)
    q, bt, ctx, scale = a.pop("q"), a.pop("block_table"), a.pop("context_lengths"), a.pop("scale")
    return pkv.decode_gqa(q, c, bt, ctx, scale, **a)


@pytest.mark.parametrize("over,match", [
    (dict(q=torch.zeros(B, HQ, D, dtype=torch.float32)), "q: dtype"),
    (dict(q=torch.zeros(B, HQ, 64, dtype=torch.bfloat16)), "q: shape"),
    (dict(q=torch.zeros(B, 7, D, dtype=torch.bfloat16)), "not a multiple"),
    (dict(q=torch.zeros(B + 1, HQ, D, dtype=torch.bfloat16)), "one row per sequence"),
    (dict(q=torch.zeros(HQ, B, D, dtype=torch.bfloat16).transpose(0, 1)), "contiguous"),
    (dict(block_table=torch.zeros(B, MBS, dtype=torch.int64)), "block_table: dtype"),
    (dict(block_table=torch.zeros(B + 1, MBS, dtype=torch.int32)), "block_table: shape"),
    (dict(context_lengths=torch.ones(B, dtype=torch.int64)), "context_lengths: dtype"),
    (dict(cu_q_lens=torch.zeros(B, dtype=torch.int32)), "cu_q_lens: shape"),
    (dict(out=torch.zeros(B, HQ, D - 8, dtype=torch.bfloat16)), "out: shape"),
    (dict(out=torch.zeros(B, HQ, D, dtype=torch.float16)), "out: dtype"),
    (dict(lse_out=torch.zeros(B, HQ + 1, dtype=torch.float32)), "lse_out: shape"),
    (dict(lse_out=torch.zeros(B, HQ, dtype=torch.float64)), "lse_out: dtype"),
    (dict(workspace=torch.zeros(64, dtype=torch.float32)), "workspace: dtype"),
    (dict(), "GPU memory only"),  # every shape right, but host memory
])
def test_decode_rejects_bad_arguments(over, match):
    with pytest.raises(ValueError, match=match):
        call_decode(cache(), **over)


def test_decode_with_chunks_checks_cu_q_lens_shape():
    q = torch.zeros(7, HQ, D, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU memory only"):  # 7 rows for 3 sequences is fine with cu_q_lens
        call_decode(cache(), q=q, cu_q_lens=torch.zeros(B + 1, dtype=torch.int32), max_q_len=5)
    with pytest.raises(ValueError, match="cu_q_lens: dtype"):
        call_decode(cache(), q=q, cu_q_lens=torch.zeros(B + 1, dtype=torch.int64), max_q_len=5)


@pytest.mark.parametrize("over,match", [
    (dict(k_new=torch.zeros(B, HKV, 64, dtype=torch.bfloat16)), "k_new: shape"),
    (dict(k_new=torch.zeros(B, HKV, D, dtype=torch.float32)), "k_new: dtype"),
    (dict(v_new=torch.zeros(B + 1, HKV, D, dtype=torch.bfloat16)), "v_new: shape"),
    (dict(context_lengths=torch.ones(B, dtype=torch.int64)), "context_lengths: dtype"),
    (dict(block_table=None), "block_table is required"),
    (dict(cu_q_lens=torch.zeros(B + 2, dtype=torch.int32)), "cu_q_lens: shape"),
    (dict(k_new=torch.zeros(B + 1, HKV, D, dtype=torch.bfloat16),
          v_new=torch.zeros(B + 1, HKV, D, dtype=torch.bfloat16)), "one token"),
    (dict(), "GPU memory only"),
])
def test_store_rejects_bad_arguments(over, match):
    a = dict(k_new=torch.zeros(B, HKV, D, dtype=torch.bfloat16), v_new=torch.zeros(B, HKV, D, dtype=torch.bfloat16),
             context_lengths=torch.ones(B, dtype=torch.int32), block_table=torch.zeros(B, MBS, dtype=torch.int32))
    a.update(over)
    k, v = a.pop("k_new"), a.pop("v_new")
    with pytest.raises(ValueError, match=match):
        pkv.store_c8(cache(), k, v, **a)


def test_store_slot_mapping_form():
    k = torch.zeros(5, HKV, D, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="slot_mapping: dtype"):
        pkv.store_c8(cache(), k, k, slot_mapping=torch.zeros(5, dtype=torch.int32))
    with pytest.raises(ValueError, match="slot_mapping: shape"):
        pkv.store_c8(cache(), k, k, slot_mapping=torch.zeros(4, dtype=torch.int64))
    with pytest.raises(ValueError, match="must be None"):
        pkv.store_c8(cache(), k, k, slot_mapping=torch.zeros(5, dtype=torch.int64),
                     context_lengths=torch.ones(5, dtype=torch.int32))
    with pytest.raises(ValueError, match="GPU memory only"):
        pkv.store_c8(cache(), k, k, slot_mapping=torch.zeros(5, dtype=torch.int64))


@pytest.mark.parametrize("over,match", [
    (dict(seq_offsets=torch.zeros(B, dtype=torch.int32)), "seq_offsets: dtype"),
    (dict(seq_offsets=torch.zeros(B + 1, dtype=torch.int64)), "seq_offsets: shape"),
    (dict(k_out=torch.zeros(10, dtype=torch.float32)), "k_out: dtype"),
    (dict(block_table=torch.zeros(B, MBS, dtype=torch.int64)), "block_table: dtype"),
    (dict(num_rows=3), "GPU memory only"),
])
def test_dequant_rejects_bad_arguments(over, match):
    a = dict(block_table=torch.zeros(B, MBS, dtype=torch.int32), context_lengths=torch.ones(B, dtype=torch.int32))
    a.update(over)
    bt, ctx = a.pop("block_table"), a.pop("context_lengths")
    with pytest.raises(ValueError, match=match):
        pkv.dequant(cache(), bt, ctx, **a)


def test_cache_checks_given_tensors():
    with pytest.raises(ValueError, match="cache.k: dtype"):
        pkv.Cache(0, NB, HKV, BS, D, device="cpu", k=torch.zeros(NB, HKV, BS, D, dtype=torch.uint8))
    with pytest.raises(ValueError, match="cache.v: shape"):
        pkv.Cache(0, NB, HKV, BS, D, device="cpu", v=torch.zeros(NB, HKV, BS, D, dtype=torch.int8))
    with pytest.raises(ValueError, match="cache.k_scale: shape"):
        pkv.Cache(1, NB, HKV, BS, D, device="cpu", k_scale=torch.zeros(NB, HKV, BS, dtype=torch.float32))


def test_mla_rejects_bad_arguments():
    c = pkv.MLACache(NB, BS, device="cpu")
    ql = torch.zeros(B, 16, 512, dtype=torch.bfloat16)
    qr = torch.zeros(B, 16, 64, dtype=torch.bfloat16)
    bt = torch.zeros(B, MBS, dtype=torch.int32)
    ctx = torch.ones(B, dtype=torch.int32)
    with pytest.raises(ValueError, match="q_rope: shape"):
        pkv.mla_decode(ql, qr[:, :8].contiguous(), c, bt, ctx, 0.1)
    with pytest.raises(ValueError, match="q_latent: shape"):
        pkv.mla_decode(ql[..., :256].contiguous(), qr, c, bt, ctx, 0.1)
    with pytest.raises(ValueError, match="out: shape"):
        pkv.mla_decode(ql, qr, c, bt, ctx, 0.1, out=torch.zeros(B, 16, 256, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="context_lengths: dtype"):
        pkv.mla_decode(ql, qr, c, bt, ctx.long(), 0.1)
    with pytest.raises(ValueError, match="GPU memory only"):
        pkv.mla_decode(ql, qr, c, bt, ctx, 0.1)
    lat = torch.zeros(B, 512, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="rope_new: shape"):
        pkv.mla_store_c8(c, lat, torch.zeros(B, 32, dtype=torch.bfloat16), context_lengths=ctx, block_table=bt)
    with pytest.raises(ValueError, match="GPU memory only"):
        pkv.mla_store_c8(c, lat, torch.zeros(B, 64, dtype=torch.bfloat16), context_lengths=ctx, block_table=bt)
