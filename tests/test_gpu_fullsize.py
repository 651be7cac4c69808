"""Parity at the benchmark workloads' full sizes, in the launch configuration bench.py times
(default split plan).  The oracle recomputes the store and the attention of sampled sequences
from the same seeded bf16 inputs; the GPU results for those sequences must match (codes and
scales bit-exact over every page of the sequence, attention within tolerance)."""
import numpy as np
import pytest
import torch

import gen
import paged_kv_cache_c8_amd as pkv
from tests.gpu_harness import Run, lse_bar, oracle_run, sub_workload
from tests.helpers import attention_close, v_token_major

pytestmark = pytest.mark.gpu


def _check(idx, n_sample, kernel=0, quant_mode=None, window=0, fused=False):
    w = gen.make_config(idx, quant_mode=quant_mode)
    r = Run(w, with_oracle=False)
    r.store_prior()
    if fused:  # the decode step with its store in one call, as bench.py times it by default
        assert w.decode_only
        q = r.queries()
        kn, vn = r._decode_rows(r.k_new), r._decode_rows(r.v_new)
        lse = torch.empty((w.batch, w.num_q_heads), dtype=torch.float32, device=q.device)
        out = pkv.store_decode_gqa(q, kn, vn, r.cache, r.bt, r.ctx, 1.0 / np.sqrt(w.head_dim), lse_out=lse)
    else:
        r.store_new()
        out, lse = r.decode(kernel=kernel, window=window)
    torch.cuda.synchronize()
    rng = np.random.default_rng(100 + idx)
    sel = np.arange(w.batch) if n_sample >= w.batch else np.sort(rng.choice(w.batch, n_sample, replace=False))
    print(f"config {idx} ({w.name}): checking sequences {sel.tolist()}", flush=True)
    ws, th = sub_workload(w, sel, r.t)
    hc, (ob, o64, olse) = oracle_run(ws, th, nthreads=16, window=window)
    # cache pages of the sampled sequences
    gk, gv = r.cache.k, r.cache.v
    for j, b in enumerate(sel):
        nblk = -(-int(w.context_lengths[b]) // w.block_size)
        blks = torch.as_tensor(w.block_table[b, :nblk].astype(np.int64), device=gk.device)
        n = int(w.context_lengths[b])
        host_blks = w.block_table[b, :nblk]
        for name, g_arr, h_arr, tok_axis in (("K", gk, hc.k, 2), ("V", gv, hc.v, 2)):
            g = g_arr.index_select(0, blks).cpu()
            g = (g.view(torch.int16).numpy().view(np.uint16) if w.quant_mode == 2 else g.numpy())
            h = h_arr[host_blks]
            if name == "V":
                g, h = v_token_major(g, w.block_size), v_token_major(h, w.block_size)
            # flatten the block/slot axes to positions and keep the defined ones
            g = np.moveaxis(g, tok_axis, 1).reshape(nblk * w.block_size, *np.moveaxis(g, tok_axis, 1).shape[2:])[:n]
            h = np.moveaxis(h, tok_axis, 1).reshape(nblk * w.block_size, *np.moveaxis(h, tok_axis, 1).shape[2:])[:n]
            assert np.array_equal(g, h), f"{name} codes differ for sequence {b}"
        if w.quant_mode == 3:  # static inputs, unchanged by the store
            assert np.array_equal(r.cache.k_scale.cpu().numpy(), hc.k_scale)
        if w.quant_mode == 0:
            for g_s, h_s in ((r.cache.k_scale, hc.k_scale), (r.cache.v_scale, hc.v_scale)):
                g = g_s.index_select(0, blks).cpu().numpy().transpose(0, 2, 1).reshape(-1, w.num_kv_heads)[:n]
                h = h_s[host_blks].transpose(0, 2, 1).reshape(-1, w.num_kv_heads)[:n]
                assert np.array_equal(g.view(np.uint32), h.view(np.uint32))
        elif w.quant_mode == 1:
            for g_s, h_s in ((r.cache.k_scale, hc.k_scale), (r.cache.v_scale, hc.v_scale)):
                g = g_s.index_select(0, blks).cpu().numpy()
                assert np.array_equal(g.view(np.uint32), h_s[host_blks].view(np.uint32))
    # attention rows of the sampled sequences
    if w.decode_only:
        rows = sel
    else:
        cu = w.cu_q_lens
        rows = np.concatenate([np.arange(cu[b], cu[b + 1]) for b in sel])
    got = out[torch.as_tensor(rows, device=out.device)].float().cpu().numpy().astype(np.float64)
    max_abs, rel, elem_ok = attention_close(got, o64)
    print(f"config {idx}: max_abs={max_abs:.3e} rel={rel:.3e}", flush=True)
    assert max_abs <= 1e-2 and rel <= 1e-2 and elem_ok
    gl = lse[torch.as_tensor(rows, device=lse.device)].cpu().numpy().astype(np.float64)
    slack = lse_bar(hc, th["q"], ws, 1.0 / np.sqrt(w.head_dim))
    fin = np.isfinite(olse)
    assert np.array_equal(np.isfinite(gl), fin)
    tol = np.broadcast_to(1e-4 + 1e-5 * np.abs(np.where(fin, olse, 0.0)) + slack, olse.shape)
    assert np.all(np.abs(gl[fin] - olse[fin]) <= tol[fin])


def test_qwen3_8b_step_with_store_full():
    """The benchmark's default step: every sequence's new token stored by the decode call itself."""
    _check(1, 32, fused=True)


def test_long_context_step_with_store_sampled():
    _check(2, 2, fused=True)


def test_qwen3_8b_decode_full():
    _check(1, 32)


def test_long_context_decode_sampled():
    _check(2, 2)


def test_bf16_large_batch_sampled():
    _check(3, 24)


def test_chunked_per_block_sampled():
    _check(4, 12)


@pytest.mark.parametrize("idx,n_sample", [(1, 32), (2, 2), (4, 12)])
def test_int8_score_kernel_full_sizes(idx, n_sample):
    _check(idx, n_sample, kernel=3)


def test_per_channel_full_sizes():
    """Static per-channel scales (mode 3) at the Qwen3-8B and long-context decodes' full sizes."""
    _check(1, 32, quant_mode=3)
    _check(2, 2, quant_mode=3)


def test_sliding_window_full_sizes():
    """Sliding windows at the Qwen3-8B and long-context decodes' full sizes, with windows
    (1024 and 32768 tokens) shorter than most of their sequences."""
    _check(1, 32, window=1024)
    _check(2, 2, window=32768)


def test_bf16_balanced_matches_fixed_splits_everywhere():
    """The bf16 large-batch decode at full size: the balanced partition (the default plan here)
    against fixed 4096-key splits on every output element of every sequence and head, within the
    bound two split plans can differ by (bf16 weights against different running maxima; bf16
    output), and the lse within 1e-5 relative."""
    w = gen.make_config(3)
    r = Run(w, with_oracle=False)
    r.store_prior()
    r.store_new()
    bal, lb = r.decode()
    fixed, lf = r.decode(split_tokens=4096)
    torch.cuda.synchronize()
    a, b = fixed.float(), bal.float()
    bound = a.abs() * 2.0 ** -7 + 2.0 ** -10 * float(a.abs().max())
    excess = ((a - b).abs() - bound).max()
    print(f"{w.name}: balanced vs fixed, largest excess over the bound {float(excess):.3e}", flush=True)
    assert bool(((a - b).abs() <= bound).all()), float(excess)
    assert torch.allclose(lb, lf, rtol=1e-5, atol=1e-5)
