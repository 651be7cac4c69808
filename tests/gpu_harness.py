"""Helpers shared by the GPU parity tests: run a workload through libpkv and through the oracle on
the same seeded inputs, then compare.

Inputs come from ``gen`` (drawn on the GPU, copied to the host for the oracle); the oracle never
sees anything the HIP path produced.
"""
from __future__ import annotations

import numpy as np
import torch

import gen
import oracle
import paged_kv_cache_c8_amd as pkv
from tests.helpers import attention_close, v_token_major


def bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def i32(x, dev):
    return torch.as_tensor(np.ascontiguousarray(x, dtype=np.int32), device=dev)


class Run:
    """One workload stored into a GPU cache (prefill of the prior tokens, then the new tokens) and,
    when ``with_oracle``, into an oracle host cache through the same two calls."""

    def __init__(self, w: gen.Workload, dev="cuda", with_oracle=True, tensors=None, fill=0):
        self.w = w
        self.dev = torch.device(dev)
        self.t = tensors if tensors is not None else gen.gen_tensors(w, device=self.dev)
        self.cache = pkv.Cache(w.quant_mode, w.num_blocks, w.num_kv_heads, w.block_size, w.head_dim,
                               device=self.dev)
        if fill:
            self.cache.k.fill_(fill)
            self.cache.v.fill_(fill)
        self.bt = i32(w.block_table, self.dev)
        self.ctx = i32(w.context_lengths, self.dev)
        self.prior = i32(w.prior_lengths, self.dev)
        self.cu_prior = i32(w.cu_prior, self.dev)
        self.cu_q = None if w.decode_only else i32(w.cu_q_lens, self.dev)
        self.k_prior, self.k_new = gen.split_prior_new(w, self.t["k_all"])
        self.v_prior, self.v_new = gen.split_prior_new(w, self.t["v_all"])
        self.hc = None
        if with_oracle:
            self.hc = oracle.HostCache(w.quant_mode, w.num_blocks, w.num_kv_heads, w.block_size, w.head_dim,
                                       fill=fill)
        if w.quant_mode == 3:  # static per-channel scales: the same inputs for both sides
            self.cache.k_scale.copy_(self.t["k_scale"])
            self.cache.v_scale.copy_(self.t["v_scale"])
            if self.hc is not None:
                self.hc.k_scale[...] = self.t["k_scale"].cpu().numpy()
                self.hc.v_scale[...] = self.t["v_scale"].cpu().numpy()

    def store_prior(self):
        w = self.w
        if int(w.prior_lengths.sum()) > 0:
            pkv.store_c8(self.cache, self.k_prior, self.v_prior, cu_q_lens=self.cu_prior,
                         context_lengths=self.prior, block_table=self.bt,
                         max_q_len=int(w.prior_lengths.max()))
            if self.hc is not None:
                oracle.store(self.hc, bits(self.k_prior), bits(self.v_prior),
                             cu_q_lens=w.cu_prior.astype(np.int32), context_lengths=w.prior_lengths,
                             block_table=w.block_table)

    def store_new(self):
        w = self.w
        if w.num_new_tokens == 0 and w.decode_only:
            pass
        if w.decode_only:
            # one new token per sequence; inactive (ctx 0) sequences get a zero row that is skipped
            kn, vn = self._decode_rows(self.k_new), self._decode_rows(self.v_new)
            pkv.store_c8(self.cache, kn, vn, context_lengths=self.ctx, block_table=self.bt)
            if self.hc is not None:
                oracle.store(self.hc, bits(kn), bits(vn), context_lengths=w.context_lengths,
                             block_table=w.block_table)
        else:
            pkv.store_c8(self.cache, self.k_new, self.v_new, cu_q_lens=self.cu_q, context_lengths=self.ctx,
                         block_table=self.bt, max_q_len=w.max_q_len)
            if self.hc is not None:
                oracle.store(self.hc, bits(self.k_new), bits(self.v_new), cu_q_lens=w.cu_q_lens,
                             context_lengths=w.context_lengths, block_table=w.block_table)

    def _decode_rows(self, new):
        """[B, Hkv, D] rows for a decode batch (zero rows for sequences without a new token)."""
        w = self.w
        if w.num_new_tokens == w.batch:
            return new
        rows = torch.zeros((w.batch, w.num_kv_heads, w.head_dim), dtype=new.dtype, device=new.device)
        has = torch.as_tensor(np.nonzero(w.q_lens)[0], device=new.device)
        rows[has] = new
        return rows

    def queries(self):
        w = self.w
        if w.decode_only and w.num_new_tokens != w.batch:
            q = torch.zeros((w.batch, w.num_q_heads, w.head_dim), dtype=torch.bfloat16, device=self.dev)
            has = torch.as_tensor(np.nonzero(w.q_lens)[0], device=self.dev)
            q[has] = self.t["q"]
            return q
        return self.t["q"]

    def decode(self, scale=None, **kw):
        w = self.w
        if scale is None:
            scale = 1.0 / np.sqrt(w.head_dim)
        self.last_scale = float(np.float32(scale))
        q = self.queries()
        lse = torch.full((q.shape[0], w.num_q_heads), 7.0, dtype=torch.float32, device=self.dev)
        out = pkv.decode_gqa(q, self.cache, self.bt, self.ctx, scale, cu_q_lens=self.cu_q,
                             max_q_len=w.max_q_len, lse_out=lse, **kw)
        return out, lse

    def oracle_decode(self, scale=None, nthreads=8, window=0):
        w = self.w
        if scale is None:
            scale = 1.0 / np.sqrt(w.head_dim)
        return oracle.decode(self.hc, bits(self.queries()), w.num_q_heads, w.block_table, w.context_lengths,
                             scale, cu_q_lens=None if w.decode_only else w.cu_q_lens, nthreads=nthreads,
                             window=window)

    # ------------------------------------------------------------------------------ checks
    def assert_cache_equal(self):
        torch.cuda.synchronize()
        k = self.cache.k.cpu()
        v = self.cache.v.cpu()
        if self.w.quant_mode == 2:
            k = k.view(torch.int16).numpy().view(np.uint16)
            v = v.view(torch.int16).numpy().view(np.uint16)
        else:
            k, v = k.numpy(), v.numpy()
        # only slots that hold a position of some sequence are defined
        mask = self.defined_slots()
        bs = self.w.block_size
        for name, got, want in (("K", k, self.hc.k), ("V", v_token_major(v, bs), v_token_major(self.hc.v, bs))):
            diff = (got != want)[mask]
            assert not diff.any(), f"{name} codes differ at {int(diff.sum())} elements"
        if self.w.quant_mode not in (2, 3):  # mode 3 scales are inputs, never written
            for name, got, want in (("K scale", self.cache.k_scale, self.hc.k_scale),
                                    ("V scale", self.cache.v_scale, self.hc.v_scale)):
                g = got.cpu().numpy().view(np.uint32)
                wv = want.view(np.uint32)
                if self.w.quant_mode == 0:
                    g, wv = g[mask[..., 0]], wv[mask[..., 0]]
                else:
                    bm = mask[..., 0].any(axis=2)
                    g, wv = g[bm], wv[bm]
                assert np.array_equal(g, wv), f"{name} differs"

    def defined_slots(self):
        """bool [NB, Hkv, BS, D] of cache slots that hold a position < ctx of some sequence."""
        w = self.w
        m = np.zeros((w.num_blocks, w.block_size), bool)
        for b in range(w.batch):
            for p in range(int(w.context_lengths[b])):
                m[w.block_table[b, p // w.block_size], p % w.block_size] = True
        return np.broadcast_to(m[:, None, :, None], (w.num_blocks, w.num_kv_heads, w.block_size, w.head_dim))

    def assert_decode_close(self, out, lse, ref=None, atol=1e-2, rtol=1e-2, scale=None):
        """Attention within the bar; lse within lse_bar.  ``scale``: the softmax scale of the GPU
        call (default: the one the last ``decode`` used; the oracle result ``ref`` must be for the
        same scale)."""
        torch.cuda.synchronize()
        if scale is None:
            scale = getattr(self, "last_scale", 1.0 / np.sqrt(self.w.head_dim))
        ob, o64, olse = ref if ref is not None else self.oracle_decode(scale=scale)
        got = out.float().cpu().numpy().astype(np.float64)
        max_abs, rel, elem_ok = attention_close(got, o64, atol, rtol)
        print(f"[{self.w.name}] attention vs oracle: max_abs={max_abs:.2e} rel={rel:.2e}", flush=True)
        assert max_abs <= atol and rel <= rtol and elem_ok, (max_abs, rel, elem_ok)
        gl = lse.cpu().numpy().astype(np.float64)
        fin = np.isfinite(olse)
        assert np.array_equal(np.isfinite(gl), fin)
        assert np.all(gl[~fin] == -np.inf)
        if fin.any():
            tol = 1e-4 + 1e-5 * np.abs(np.where(fin, olse, 0.0)) + lse_bar(self.hc, bits(self.queries()), self.w, scale)
            err = np.abs(gl[fin] - olse[fin])
            print(f"[{self.w.name}] lse vs oracle: max_err={float(err.max()):.2e} (bar >= {float(tol[fin].min()):.2e})",
                  flush=True)
            assert np.all(err <= tol[fin]), float(err.max())
        return max_abs, rel


def sub_workload(w: gen.Workload, sel, t):
    """The sequences ``sel`` of ``w`` as their own workload (same pool and physical blocks), with
    their rows of the drawn tensors copied to the host as bf16 bits."""
    import dataclasses

    sel = np.asarray(sel)
    ws = dataclasses.replace(w, batch=len(sel), context_lengths=w.context_lengths[sel].copy(),
                             q_lens=w.q_lens[sel].copy(), block_table=w.block_table[sel].copy())
    cu_ctx, cu_q = w.cu_context, w.cu_q_lens
    kv_idx = np.concatenate([np.arange(cu_ctx[b], cu_ctx[b + 1]) for b in sel])
    if w.decode_only:
        q_idx = sel
    else:
        q_idx = np.concatenate([np.arange(cu_q[b], cu_q[b + 1]) for b in sel])
    dev = t["q"].device
    th = {
        "q": bits(t["q"].index_select(0, torch.as_tensor(q_idx, device=dev))),
        "k_all": bits(t["k_all"].index_select(0, torch.as_tensor(kv_idx, device=dev))),
        "v_all": bits(t["v_all"].index_select(0, torch.as_tensor(kv_idx, device=dev))),
    }
    if "k_scale" in t:  # static per-channel scales: the same inputs
        th["k_scale"], th["v_scale"] = t["k_scale"].cpu().numpy(), t["v_scale"].cpu().numpy()
    return ws, th


def oracle_run(ws: gen.Workload, th, nthreads=8, window=0):
    """Prefill store of the prior tokens, store of the new tokens, fp64 decode - all in the oracle."""
    hc = oracle.HostCache(ws.quant_mode, ws.num_blocks, ws.num_kv_heads, ws.block_size, ws.head_dim)
    if ws.quant_mode == 3:
        hc.k_scale[...] = th["k_scale"]
        hc.v_scale[...] = th["v_scale"]
    cu_ctx = ws.cu_context
    prior = ws.prior_lengths
    pri_idx = np.concatenate([np.arange(cu_ctx[b], cu_ctx[b] + prior[b]) for b in range(ws.batch)] + [[]]).astype(np.int64)
    new_idx = np.concatenate([np.arange(cu_ctx[b] + prior[b], cu_ctx[b + 1]) for b in range(ws.batch)] + [[]]).astype(np.int64)
    if len(pri_idx):
        oracle.store(hc, th["k_all"][pri_idx], th["v_all"][pri_idx], cu_q_lens=ws.cu_prior.astype(np.int32),
                     context_lengths=prior, block_table=ws.block_table)
    cu = None if ws.decode_only else ws.cu_q_lens
    oracle.store(hc, th["k_all"][new_idx], th["v_all"][new_idx], cu_q_lens=cu if cu is not None else None,
                 context_lengths=ws.context_lengths, block_table=ws.block_table)
    scale = 1.0 / np.sqrt(ws.head_dim)
    res = oracle.decode(hc, th["q"], ws.num_q_heads, ws.block_table, ws.context_lengths, scale,
                        cu_q_lens=cu, nthreads=nthreads, window=window)
    return hc, res


def key_values(hc, w, b, h):
    """K of sequence b, KV head h, as exact float64 values [ctx, D] (codes times their scales, or
    the stored bf16 values)."""
    from tests.helpers import bits_to_f32

    n = int(w.context_lengths[b])
    pos = np.arange(n)
    blk = w.block_table[b, pos // w.block_size]
    off = pos % w.block_size
    k = hc.k[blk, h, off, :]  # [n, D]
    if w.quant_mode == 2:
        return bits_to_f32(k).astype(np.float64)
    k = k.astype(np.float64)
    if w.quant_mode == 0:
        return k * hc.k_scale[blk, h, off][:, None]
    if w.quant_mode == 1:
        return k * hc.k_scale[blk, h][:, None]
    return k * hc.k_scale[h][None].astype(np.float64)


def lse_bar(hc, q_bits, w, scale):
    """The part of the lse tolerance that grows with the logits, per (query row, head): the error
    bound of evaluating the definition in fp32 arithmetic, D * 2^-24 * |scale| * max_t
    sum_d |q_d| |K_td| (a D-term dot product in fp32; every key of the sequence is taken, an upper
    bound of the row's visible keys).  It depends on the inputs only, not on how a kernel forms
    its logits."""
    from tests.helpers import bits_to_f32

    q = np.abs(bits_to_f32(q_bits).astype(np.float64))  # [Tq, Hq, D]
    g = w.num_q_heads // w.num_kv_heads
    out = np.zeros(q.shape[:2])
    row0 = 0
    for b in range(w.batch):
        nq = 1 if w.decode_only else int(w.q_lens[b])
        rows = slice(row0, row0 + nq)
        row0 += nq
        if int(w.context_lengths[b]) == 0 or nq == 0:
            continue
        for h in range(w.num_kv_heads):
            kv = np.abs(key_values(hc, w, b, h))  # [n, D]
            qq = q[rows, h * g:(h + 1) * g, :].reshape(-1, w.head_dim)
            out[rows, h * g:(h + 1) * g] = (qq @ kv.T).max(axis=1).reshape(nq, g)
    return w.head_dim * 2.0 ** -24 * abs(scale) * out
