"""GPU parity of the paged MLA (latent cache) path with the oracle: the store bit-exact (codes and
scales), the decode within 1e-2 (max abs and norm-relative) and its lse within 1e-4 + 1e-5|lse|
plus the error bound of an fp32 evaluation of the logits (lse_bar)."""
import numpy as np
import pytest
import torch

import gen
import oracle
import paged_kv_cache_c8_amd as pkv
from tests.helpers import attention_close, bits_to_f32

pytestmark = pytest.mark.gpu

DEV = "cuda"


def bits(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


class MlaRun:
    """One MLA workload on the GPU: the prior tokens stored in one prefill-style call, then one new
    token per sequence (the decode step's store), then the decode."""

    def __init__(self, w):
        self.w = w
        self.t = gen.gen_mla_tensors(w, device=DEV)
        self.cache = pkv.MLACache(w.num_blocks, w.block_size, device=DEV)
        self.bt = torch.as_tensor(w.block_table, device=DEV)
        self.ctx = torch.as_tensor(w.context_lengths, device=DEV)

    def store(self):
        w, t = self.w, self.t
        prior = w.prior_lengths
        cu_ctx = w.cu_context
        pri = np.concatenate([np.arange(cu_ctx[b], cu_ctx[b] + prior[b]) for b in range(w.batch)] + [[]]).astype(np.int64)
        new = np.array([cu_ctx[b + 1] - 1 for b in range(w.batch) if w.context_lengths[b] > 0], np.int64)
        pi = torch.as_tensor(pri, device=DEV)
        cu_p = np.zeros(w.batch + 1, np.int32)
        cu_p[1:] = np.cumsum(prior)
        if len(pri):
            pkv.mla_store_c8(self.cache, t["latent_all"].index_select(0, pi), t["rope_all"].index_select(0, pi),
                             cu_q_lens=torch.as_tensor(cu_p, device=DEV),
                             context_lengths=torch.as_tensor(prior, device=DEV), block_table=self.bt)
        # decode step: one token per sequence (rows of empty sequences are never read)
        rows = np.array([cu_ctx[b + 1] - 1 if w.context_lengths[b] > 0 else 0 for b in range(w.batch)], np.int64)
        ri = torch.as_tensor(rows, device=DEV)
        lat = t["latent_all"].index_select(0, ri).contiguous() if w.batch else t["latent_all"][:0]
        rot = t["rope_all"].index_select(0, ri).contiguous() if w.batch else t["rope_all"][:0]
        pkv.mla_store_c8(self.cache, lat, rot, context_lengths=self.ctx, block_table=self.bt)
        return new

    def decode(self, split_tokens=0, scale=None):
        w = self.w
        lse = torch.full((w.batch, w.num_heads), 7.0, dtype=torch.float32, device=DEV)
        out = pkv.mla_decode(self.t["q_latent"], self.t["q_rope"], self.cache, self.bt, self.ctx,
                             w.softmax_scale if scale is None else scale, lse_out=lse, split_tokens=split_tokens)
        return out, lse


def oracle_cache(w, t, seqs=None):
    """The oracle's cache for the sequences ``seqs`` (all by default), stored in one call."""
    c = oracle.MLAHostCache(w.num_blocks, w.block_size, w.latent_dim, w.rope_dim)
    seqs = range(w.batch) if seqs is None else seqs
    cu_ctx = w.cu_context
    idx = np.concatenate([np.arange(cu_ctx[b], cu_ctx[b + 1]) for b in seqs] + [[]]).astype(np.int64)
    ctx = w.context_lengths[list(seqs)]
    cu = np.zeros(len(ctx) + 1, np.int32)
    cu[1:] = np.cumsum(ctx)
    ii = torch.as_tensor(idx, device=t["latent_all"].device)
    oracle.mla_store(c, bits(t["latent_all"].index_select(0, ii)), bits(t["rope_all"].index_select(0, ii)),
                     cu_q_lens=cu, context_lengths=ctx, block_table=w.block_table[list(seqs)])
    return c


def lse_bar(hc, q_lat_bits, q_rope_bits, w, seqs, scale):
    """The part of the lse tolerance that grows with the logits, per (sequence, head): the error
    bound of evaluating the definition in fp32, (512 + 64) * 2^-24 * |scale| * max_t (sum |q_c| |c_t|
    + sum |q_r| |r_t|) over the sequence's keys.  It depends on the inputs only."""
    out = np.zeros((len(seqs), w.num_heads))
    for j, b in enumerate(seqs):
        n = int(w.context_lengths[b])
        if n == 0:
            continue
        pos = np.arange(n)
        blk = w.block_table[b, pos // w.block_size]
        off = pos % w.block_size
        c = np.abs(hc.latent[blk, off].astype(np.float64)) * hc.latent_scale[blk, off][:, None]
        r = np.abs(hc.rope[blk, off].astype(np.float64)) * hc.rope_scale[blk, off][:, None]
        qc = np.abs(bits_to_f32(q_lat_bits[j]).astype(np.float64))   # [H, 512]
        qr = np.abs(bits_to_f32(q_rope_bits[j]).astype(np.float64))  # [H, 64]
        out[j] = (qc @ c.T + qr @ r.T).max(axis=1)
    return (w.latent_dim + w.rope_dim) * 2.0 ** -24 * abs(scale) * out


def check_decode(r, out, lse, seqs, hc=None):
    w = r.w
    if hc is None:
        hc = oracle_cache(w, r.t, seqs)
    sub_bt = w.block_table[list(seqs)]
    qi = torch.as_tensor(np.asarray(seqs, np.int64), device=DEV)
    ql, qr = bits(r.t["q_latent"].index_select(0, qi)), bits(r.t["q_rope"].index_select(0, qi))
    _, o64, olse = oracle.mla_decode(hc, ql, qr, sub_bt, w.context_lengths[list(seqs)], w.softmax_scale,
                                     nthreads=8)
    got = out.index_select(0, qi).float().cpu().numpy().astype(np.float64)
    max_abs, rel, elem_ok = attention_close(got, o64)
    print(f"{w.name}: max_abs={max_abs:.3e} rel={rel:.3e}", flush=True)
    assert max_abs <= 1e-2 and rel <= 1e-2 and elem_ok
    gl = lse.index_select(0, qi).cpu().numpy().astype(np.float64)
    fin = np.isfinite(olse)
    assert np.array_equal(np.isfinite(gl), fin)
    tol = 1e-4 + 1e-5 * np.abs(np.where(fin, olse, 0.0)) + lse_bar(hc, ql, qr, w, seqs, w.softmax_scale)
    if fin.any():
        print(f"{w.name}: lse max_err={float(np.abs(gl[fin] - olse[fin]).max()):.2e}", flush=True)
    assert np.all(np.abs(gl[fin] - olse[fin]) <= tol[fin])
    empty = ~fin
    assert np.all(got[empty] == 0)


def test_store_bit_exact():
    w = gen.mla_workload("store", batch=4, num_heads=16, block_size=16, context_lengths=[1, 37, 100, 16], seed=1)
    r = MlaRun(w)
    r.store()
    torch.cuda.synchronize()
    hc = oracle_cache(w, r.t)
    assert np.array_equal(r.cache.latent.cpu().numpy(), hc.latent)
    assert np.array_equal(r.cache.rope.cpu().numpy(), hc.rope)
    assert np.array_equal(r.cache.latent_scale.cpu().numpy().view(np.uint32), hc.latent_scale.view(np.uint32))
    assert np.array_equal(r.cache.rope_scale.cpu().numpy().view(np.uint32), hc.rope_scale.view(np.uint32))


def test_store_slot_mapping_and_skips():
    w = gen.mla_workload("slots", batch=2, num_heads=16, block_size=32, context_lengths=[40, 9], seed=2)
    t = gen.gen_mla_tensors(w, device=DEV)
    slots = []
    for b in range(w.batch):
        for p in range(int(w.context_lengths[b])):
            slots.append(int(w.block_table[b, p // 32]) * 32 + p % 32)
    sm = np.array(slots[:20] + [-1, -1] + slots[20:], np.int64)
    lat = torch.cat([t["latent_all"][:20], torch.ones(2, 512, dtype=torch.bfloat16, device=DEV), t["latent_all"][20:]])
    rot = torch.cat([t["rope_all"][:20], torch.ones(2, 64, dtype=torch.bfloat16, device=DEV), t["rope_all"][20:]])
    c = pkv.MLACache(w.num_blocks, 32, device=DEV)
    pkv.mla_store_c8(c, lat.contiguous(), rot.contiguous(), slot_mapping=torch.as_tensor(sm, device=DEV))
    torch.cuda.synchronize()
    hc = oracle_cache(w, t)
    assert np.array_equal(c.latent.cpu().numpy(), hc.latent) and np.array_equal(c.rope.cpu().numpy(), hc.rope)
    assert np.array_equal(c.latent_scale.cpu().numpy().view(np.uint32), hc.latent_scale.view(np.uint32))
    assert np.array_equal(c.rope_scale.cpu().numpy().view(np.uint32), hc.rope_scale.view(np.uint32))


CASES = [
    # block size, heads, context lengths, split_tokens (0: the library's plan)
    (16, 16, [37, 100], 0),
    (16, 16, [37, 100], 64),
    (64, 16, [1, 63, 64, 65, 130, 1000], 0),
    (64, 16, [1, 63, 64, 65, 130, 1000], 100000),
    (16, 8, [300, 17], 128),
    (32, 32, [700, 5], 256),
    (128, 128, [513, 129], 0),
    (16, 16, [0, 50, 0], 0),
    (16, 16, [0, 50, 0], 64),
    (128, 24, [2000], 192),
]


@pytest.mark.parametrize("bs,heads,ctx,split", CASES)
def test_decode_matches_oracle(bs, heads, ctx, split):
    w = gen.mla_workload(f"mla-{bs}-{heads}-{len(ctx)}-{split}", batch=len(ctx), num_heads=heads, block_size=bs,
                         context_lengths=ctx, seed=bs + heads + split, softmax_scale=1.0 / np.sqrt(192.0))
    r = MlaRun(w)
    r.store()
    out, lse = r.decode(split_tokens=split)
    torch.cuda.synchronize()
    check_decode(r, out, lse, list(range(w.batch)))


def test_decode_split_count_agreement_and_determinism():
    """One split against many: they differ only in rounding (the weights enter the P.V products
    as fp16, relative rounding <= 2^-11 against a running max that depends on the split
    boundaries; the output is rounded to bf16, one step <= 2^-7 relative), and the lse is fp32; a
    repeated call is bit-identical."""
    w = gen.mla_workload("splits", batch=3, num_heads=16, block_size=64, context_lengths=[900, 2000, 64], seed=9)
    r = MlaRun(w)
    r.store()
    o1, l1 = r.decode(split_tokens=100000)
    o2, l2 = r.decode(split_tokens=128)
    o3, l3 = r.decode(split_tokens=128)
    torch.cuda.synchronize()
    assert torch.equal(o2, o3) and torch.equal(l2, l3)
    a, b = o1.float(), o2.float()
    bound = a.abs() * 2.0 ** -7 + 2.0 ** -10 * float(a.abs().max())
    assert bool(((a - b).abs() <= bound).all()), float(((a - b).abs() - bound).max())
    assert torch.allclose(l1, l2, rtol=1e-5, atol=1e-5)


def test_decode_negative_and_zero_scale():
    w = gen.mla_workload("scale", batch=2, num_heads=16, block_size=16, context_lengths=[33, 70], seed=12)
    r = MlaRun(w)
    r.store()
    for s in (-0.05, 0.0):
        out, lse = r.decode(scale=s)
        torch.cuda.synchronize()
        w.softmax_scale = s
        check_decode(r, out, lse, [0, 1])


def test_deepseek_shaped_decode_sampled():
    """The DeepSeek-V3-shaped MLA decode at full size, in the default plan: the store bit-exact over
    the sampled sequences' pages, their attention against the oracle."""
    w = gen.make_mla_config(1)
    r = MlaRun(w)
    r.store()
    out, lse = r.decode()
    torch.cuda.synchronize()
    seqs = sorted(np.random.default_rng(5).choice(w.batch, 4, replace=False).tolist())
    print(f"{w.name}: checking sequences {seqs}", flush=True)
    hc = oracle_cache(w, r.t, seqs)
    gl, gr = r.cache.latent.cpu().numpy(), r.cache.rope.cpu().numpy()
    gls, grs = r.cache.latent_scale.cpu().numpy(), r.cache.rope_scale.cpu().numpy()
    for b in seqs:
        used = w.block_table[b, : -(-int(w.context_lengths[b]) // w.block_size)]
        n = int(w.context_lengths[b])
        flat = lambda a: a[used].reshape(len(used) * w.block_size, *a.shape[2:])[:n]
        assert np.array_equal(flat(gl), flat(hc.latent)) and np.array_equal(flat(gr), flat(hc.rope))
        assert np.array_equal(flat(gls).view(np.uint32), flat(hc.latent_scale).view(np.uint32))
        assert np.array_equal(flat(grs).view(np.uint32), flat(hc.rope_scale).view(np.uint32))
    check_decode(r, out, lse, seqs, hc=hc)


def test_balanced_partition_garbage_workspace_and_agreement():
    """The default plan (a balanced partition of every key block over the GPU's resident
    workgroups) with a workspace full of 0xFF bytes (NaN partials, segment records of -1): items
    of one segment, of many segments and with no key are all served from what the call itself
    writes; the result matches the oracle, agrees with one split per sequence to rounding, and a
    repeated call is bit-identical."""
    ctx = [0, 1, 64, 65, 3000, 129, 0, 7000, 640, 2]
    w = gen.mla_workload("balanced", batch=len(ctx), num_heads=32, block_size=32, context_lengths=ctx, seed=31,
                         softmax_scale=1.0 / np.sqrt(192.0))
    r = MlaRun(w)
    r.store()
    plan = pkv.mla_decode_plan(w.batch, w.num_heads, w.max_blocks_per_seq, w.block_size)
    assert plan["split_tokens"] == 0 and plan["num_splits"] >= 256, plan  # the balanced partition
    need = pkv.mla_decode_workspace_size(w.batch, w.num_heads, w.max_blocks_per_seq, w.block_size)
    ws = torch.full((need,), 255, dtype=torch.uint8, device=DEV)
    bt, cl = r.bt, r.ctx

    def run(split):
        lse = torch.full((w.batch, w.num_heads), 7.0, dtype=torch.float32, device=DEV)
        o = pkv.mla_decode(r.t["q_latent"], r.t["q_rope"], r.cache, bt, cl, w.softmax_scale, lse_out=lse,
                           workspace=ws if split == 0 else None, split_tokens=split)
        return o, lse

    o_b, l_b = run(0)
    torch.cuda.synchronize()
    check_decode(r, o_b, l_b, list(range(w.batch)))
    ws.fill_(255)
    o_b2, l_b2 = run(0)
    o_1, l_1 = run(100000)
    torch.cuda.synchronize()
    assert torch.equal(o_b, o_b2) and torch.equal(l_b, l_b2)
    a, b = o_1.float(), o_b.float()
    bound = a.abs() * 2.0 ** -7 + 2.0 ** -10 * float(a.abs().max())
    assert bool(((a - b).abs() <= bound).all()), float(((a - b).abs() - bound).max())
    fin = torch.isfinite(l_1)
    assert torch.equal(fin, torch.isfinite(l_b))
    assert torch.allclose(l_1[fin], l_b[fin], rtol=1e-5, atol=1e-5)


def test_many_sequences_fall_back_to_fixed_splits():
    """Items too many for a balanced partition (twice the resident workgroups or more) run one
    workgroup per item with no merge; still within the oracle's tolerance."""
    rng = np.random.default_rng(77)
    ctx = rng.integers(1, 200, size=600).tolist()
    w = gen.mla_workload("many", batch=len(ctx), num_heads=16, block_size=16, context_lengths=ctx, seed=78,
                         softmax_scale=1.0 / np.sqrt(192.0))
    plan = pkv.mla_decode_plan(w.batch, w.num_heads, w.max_blocks_per_seq, w.block_size)
    assert plan["split_tokens"] > 0, plan
    r = MlaRun(w)
    r.store()
    out, lse = r.decode()
    torch.cuda.synchronize()
    check_decode(r, out, lse, list(range(0, w.batch, 7)))


@pytest.mark.parametrize("bs", [16, 128])
def test_long_ranges_cross_page_id_chunks(bs):
    """One workgroup walks more than 128 blocks of 64 keys (its page ids come in chunks of 64
    blocks): one split over 12000- and 9000-key contexts, and fixed 8192-key splits."""
    w = gen.mla_workload(f"long-{bs}", batch=2, num_heads=16, block_size=bs, context_lengths=[12000, 9000],
                         seed=40 + bs, softmax_scale=1.0 / np.sqrt(192.0))
    r = MlaRun(w)
    r.store()
    for split in (1 << 20, 8192):
        out, lse = r.decode(split_tokens=split)
        torch.cuda.synchronize()
        check_decode(r, out, lse, [0, 1])


def _new_rows(w, t):
    """The decode step's new latent and rotary rows, one per sequence (zero rows for empty ones)."""
    cu_ctx = w.cu_context
    rows = np.array([cu_ctx[b + 1] - 1 if w.context_lengths[b] > 0 else 0 for b in range(w.batch)], np.int64)
    ri = torch.as_tensor(rows, device=DEV)
    return t["latent_all"].index_select(0, ri).contiguous(), t["rope_all"].index_select(0, ri).contiguous()


def _store_prior(r):
    w, t = r.w, r.t
    prior = w.prior_lengths
    cu_ctx = w.cu_context
    pri = np.concatenate([np.arange(cu_ctx[b], cu_ctx[b] + prior[b]) for b in range(w.batch)] + [[]]).astype(np.int64)
    if len(pri):
        pi = torch.as_tensor(pri, device=DEV)
        cu_p = np.zeros(w.batch + 1, np.int32)
        cu_p[1:] = np.cumsum(prior)
        pkv.mla_store_c8(r.cache, t["latent_all"].index_select(0, pi), t["rope_all"].index_select(0, pi),
                         cu_q_lens=torch.as_tensor(cu_p, device=DEV),
                         context_lengths=torch.as_tensor(prior, device=DEV), block_table=r.bt)


def _assert_same_cache(c1, c2):
    for name in ("latent", "rope", "latent_scale", "rope_scale"):
        a, b = getattr(c1, name), getattr(c2, name)
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), name


STEP_CASES = [
    # block size, heads, context lengths (new token at ctx - 1), split_tokens (0: the plan)
    (16, 16, [37, 100, 1, 0, 64, 65, 130, 129], 0),    # balanced, stored inside the decode
    (64, 16, [1, 63, 64, 65, 1000, 2049], 128),         # fixed splits, stored inside the decode
    (128, 16, [2000, 5000, 64], 0),
    (16, 32, [300, 17, 1], 0),                          # two head groups: a store launch first
    (32, 8, [700, 5], 256),
]


@pytest.mark.parametrize("bs,heads,ctx,split", STEP_CASES)
def test_store_decode_equals_store_then_decode(bs, heads, ctx, split):
    """pkv_mla_store_decode against pkv_mla_store_c8 + pkv_mla_decode: the cache bytes, outputs
    and lse bit for bit the same (inside the decode launch the workgroup whose keys end at the new
    position quantizes the token itself and patches its codes into the block that holds it)."""
    w = gen.mla_workload(f"mla-step-{bs}-{heads}", batch=len(ctx), num_heads=heads, block_size=bs,
                         context_lengths=ctx, seed=bs + heads + len(ctx), softmax_scale=1.0 / np.sqrt(192.0))
    fused, two = MlaRun(w), MlaRun(w)
    two.t = fused.t
    _store_prior(fused)
    two.store()
    lat, rot = _new_rows(w, fused.t)
    lse_f = torch.full((w.batch, heads), 7.0, dtype=torch.float32, device=DEV)
    out_f = pkv.mla_store_decode(fused.t["q_latent"], fused.t["q_rope"], lat, rot, fused.cache, fused.bt, fused.ctx,
                                 w.softmax_scale, lse_out=lse_f, split_tokens=split)
    out_t, lse_t = two.decode(split_tokens=split)
    torch.cuda.synchronize()
    _assert_same_cache(fused.cache, two.cache)
    assert torch.equal(out_f.view(torch.int16), out_t.view(torch.int16))
    assert torch.equal(lse_f.view(torch.int32), lse_t.view(torch.int32))


def test_store_decode_repeated_steps():
    """Several MLA decode steps in a row, each storing one more token per sequence (the new token of
    one step is an ordinary cached key of the next), against the two-call path."""
    ctx0 = np.array([100, 1023, 4000, 1, 64])
    steps = 4
    w = gen.mla_workload("mla-steps", batch=len(ctx0), num_heads=16, block_size=64,
                         context_lengths=list(ctx0 + steps - 1), seed=17, softmax_scale=1.0 / np.sqrt(192.0))
    t = gen.gen_mla_tensors(w, device=DEV)
    bt = torch.as_tensor(w.block_table, device=DEV)
    caches = [pkv.MLACache(w.num_blocks, w.block_size, device=DEV) for _ in range(2)]
    cu = w.cu_context
    rows = torch.as_tensor(np.concatenate([np.arange(cu[b], cu[b] + ctx0[b] - 1) for b in range(w.batch)]),
                           device=DEV)
    cu_p = torch.as_tensor(np.concatenate([[0], np.cumsum(ctx0 - 1)]).astype(np.int32), device=DEV)
    for c in caches:
        pkv.mla_store_c8(c, t["latent_all"].index_select(0, rows), t["rope_all"].index_select(0, rows),
                         cu_q_lens=cu_p, context_lengths=torch.as_tensor((ctx0 - 1).astype(np.int32), device=DEV),
                         block_table=bt)
    gq = torch.Generator(device=DEV).manual_seed(19)
    for step in range(steps):
        ctx = torch.as_tensor((ctx0 + step).astype(np.int32), device=DEV)
        new = torch.as_tensor(np.array([cu[b] + ctx0[b] - 1 + step for b in range(w.batch)]), device=DEV)
        lat = t["latent_all"].index_select(0, new).contiguous()
        rot = t["rope_all"].index_select(0, new).contiguous()
        ql = torch.randn((w.batch, 16, 512), generator=gq, device=DEV).to(torch.bfloat16)
        qr = torch.randn((w.batch, 16, 64), generator=gq, device=DEV).to(torch.bfloat16)
        out_f = pkv.mla_store_decode(ql, qr, lat, rot, caches[0], bt, ctx, 0.07)
        pkv.mla_store_c8(caches[1], lat, rot, context_lengths=ctx, block_table=bt)
        out_t = pkv.mla_decode(ql, qr, caches[1], bt, ctx, 0.07)
        torch.cuda.synchronize()
        assert torch.equal(out_f.view(torch.int16), out_t.view(torch.int16)), step
        _assert_same_cache(caches[0], caches[1])
