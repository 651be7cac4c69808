"""The C-ABI library loads, exports every symbol include/pkv.h declares, and rejects bad arguments
on the host before launching anything (CPU only: no compute call reaches a kernel)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pkv.h")


@pytest.fixture(scope="module")
def pkv():
    import paged_kv_cache_c8_amd as pkv

    if not os.path.exists(pkv.LIB_PATH):
        pytest.fail("libpkv.so is not built: run `python -c 'import __graft_entry__ as g; g.build()'`")
    return pkv


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_[a-z0-9_]+)\s*\(", text)))


def test_header_declarations_are_exported(pkv):
    names = declared_functions()
    assert names, "no declarations found"
    assert sorted(names) == sorted(pkv.EXPORTS)
    lib = pkv.lib()
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", pkv.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for n in names:
        assert n in exported, n


def test_status_strings_and_version(pkv):
    lib = pkv.lib()
    assert lib.pkv_version() == 100
    for s in (0, -1, -2, -3, -4):
        assert lib.pkv_status_string(s)
    assert b"UNKNOWN" in lib.pkv_status_string(-99)


def test_plan_is_deterministic_and_bounded(pkv):
    p = pkv.decode_plan(32, 32, 8, 128, 256, 16, 1, 0)
    assert p == pkv.decode_plan(32, 32, 8, 128, 256, 16, 1, 0)
    assert p["split_tokens"] % 128 == 0 and p["num_splits"] * p["split_tokens"] >= 256 * 16
    forced = pkv.decode_plan(8, 64, 8, 128, 1024, 128, 1, 0, split_tokens=1000)
    assert forced["split_tokens"] == 1024 and forced["num_splits"] == 128
    capped = pkv.decode_plan(8, 64, 8, 128, 1024, 128, 1, 0, split_tokens=100000)
    assert capped["split_tokens"] == 4096 and capped["num_splits"] == 32
    one = pkv.decode_plan(2, 8, 2, 64, 7, 16, 1, 0, split_tokens=100000)
    assert one["num_splits"] == 1
    assert pkv.decode_plan(2, 8, 2, 64, 7, 16, 1, 0)["kernel"] == 3  # int8 pages: int8 scores
    assert pkv.decode_plan(2, 8, 2, 64, 7, 16, 1, 2)["kernel"] == 2  # bf16 pages
    assert pkv.decode_plan(2, 8, 2, 64, 7, 16, 1, 2, kernel=3)["kernel"] == 2
    assert pkv.decode_plan(2, 8, 2, 64, 7, 16, 1, 0, kernel=1)["kernel"] == 1
    assert pkv.decode_plan(2, 8, 2, 64, 7, 16, 1, 0, kernel=2)["kernel"] == 2
    # the tile kernel: int8 pages, head_dim 128, no window; one pass over each tile's keys with no
    # workspace where the tiles fill the GPU twice (prompts), whatever the context; otherwise, and
    # past 4096 keys, key splits of 4096 (forced: rounded up to 64, at most 4096) whose partials are
    # two 64-row items per 128-row tile
    tile = pkv.decode_plan(4, 32, 8, 128, 128, 16, 2048, 0, kernel=4)
    assert tile["kernel"] == 4 and tile["num_splits"] == 1
    assert pkv.decode_plan(4, 32, 8, 128, 128, 16, 2048, 1, kernel=4)["kernel"] == 4
    assert pkv.decode_workspace_size(4, 32, _py_cache(pkv), 128, max_q_len=2048, kernel=4) == 0
    long = pkv.decode_plan(4, 32, 8, 128, 1153, 16, 2048, 0, kernel=4)  # 2048 tiles, 18448 keys
    assert long["num_splits"] == 1 and long["split_tokens"] == 18496
    assert pkv.decode_workspace_size(4, 32, _py_cache(pkv), 1153, max_q_len=2048, kernel=4) == 0
    few = pkv.decode_plan(1, 8, 8, 128, 1153, 16, 16, 0, kernel=4)  # 8 tiles
    assert few["split_tokens"] == 4096 and few["num_splits"] == 5
    one_round = pkv.decode_plan(64, 40, 8, 128, 1024, 16, 16, 1, kernel=4)  # 512 tiles: one round
    assert one_round["split_tokens"] == 4096 and one_round["num_splits"] == 4
    assert pkv.decode_workspace_size(1, 8, _py_cache(pkv), 1153, max_q_len=16, kernel=4) == \
        2 * 8 * 5 * 64 * (128 + 1) * 4
    forced = pkv.decode_plan(4, 32, 8, 128, 128, 16, 2048, 0, kernel=4, split_tokens=100)
    assert forced["split_tokens"] == 128 and forced["num_splits"] == 16
    capped = pkv.decode_plan(4, 32, 8, 128, 1153, 16, 2048, 0, kernel=4, split_tokens=100000)
    assert capped["split_tokens"] == 4096 and capped["num_splits"] == 5
    for args, kw in (((4, 32, 8, 64, 128, 16, 2048, 0), {}),          # head_dim 64
                     ((4, 32, 8, 128, 128, 16, 2048, 2), {}),         # bf16 pages
                     ((4, 32, 8, 128, 128, 16, 2048, 3), {}),         # static per-channel scales
                     ((4, 32, 8, 128, 128, 16, 2048, 0), {"window": 256}),
                     ((4, 32, 8, 128, 128, 16, 2048, 0), {"partition": 2})):
        with pytest.raises(pkv.PkvError):
            pkv.decode_plan(*args, kernel=4, **kw)
    with pytest.raises(pkv.PkvError):
        pkv.decode_plan(2, 8, 2, 128, 7, 16, 1, 0, kernel=5)


def _py_cache(pkv):
    """A Cache object describing a 128-dim int8 cache without device memory (sizes only)."""
    c = pkv.Cache.__new__(pkv.Cache)
    c.num_kv_heads, c.head_dim, c.block_size, c.quant_mode = 8, 128, 16, 0
    return c


def _cache_struct(pkv, mode=0, hd=128, bs=16, k=16, v=32, ks=64, vs=128):
    return pkv._CacheT(k, v, ks, vs, 4, 2, bs, hd, mode)


def test_store_rejects_bad_arguments(pkv):
    lib = pkv.lib()
    P = 4096  # a fake, aligned device address: never dereferenced because validation fails first
    c = _cache_struct(pkv)
    r = lambda *a: lib.pkv_store_c8(*a)
    assert r(None, P, P, 1, None, None, P, P, 1, 1, 1, 0, None) == -1          # no cache
    assert r(ctypes.byref(c), P, P, 1, None, None, P, P, 1, 1, 1, 1, None) == -1  # mode mismatch
    assert r(ctypes.byref(c), P, P, -1, None, None, P, P, 1, 1, 1, 0, None) == -1  # negative tokens
    assert r(ctypes.byref(c), P, P, 0, None, None, P, P, 1, 1, 1, 0, None) == 0    # nothing to do
    assert r(ctypes.byref(c), None, P, 1, None, None, P, P, 1, 1, 1, 0, None) == -1  # no k_new
    assert r(ctypes.byref(c), P, P, 2, None, None, P, P, 1, 1, 1, 0, None) == -1   # decode: T != B
    assert r(ctypes.byref(c), P, P, 1, None, None, None, P, 1, 1, 1, 0, None) == -1  # no ctx
    bad_hd = _cache_struct(pkv, hd=96)
    assert r(ctypes.byref(bad_hd), P, P, 1, None, None, P, P, 1, 1, 1, 0, None) == -2
    bad_bs = _cache_struct(pkv, bs=24)
    assert r(ctypes.byref(bad_bs), P, P, 1, None, None, P, P, 1, 1, 1, 0, None) == -2
    per_block = _cache_struct(pkv, mode=1)
    assert r(ctypes.byref(per_block), P, P, 1, P, None, None, None, 0, 0, 1, 1, None) == -2  # slots
    misaligned = _cache_struct(pkv, k=17)
    assert r(ctypes.byref(misaligned), P, P, 1, None, None, P, P, 1, 1, 1, 0, None) == -1
    misaligned_scale = _cache_struct(pkv, ks=68)
    assert r(ctypes.byref(misaligned_scale), P, P, 1, None, None, P, P, 1, 1, 1, 0, None) == -1
    noscale = _cache_struct(pkv, ks=0)
    assert r(ctypes.byref(noscale), P, P, 1, None, None, P, P, 1, 1, 1, 0, None) == -1


def test_dequant_and_decode_reject_bad_arguments(pkv):
    lib = pkv.lib()
    P = 4096
    c = _cache_struct(pkv)
    assert lib.pkv_dequant(ctypes.byref(c), P, 1, P, None, 1, None, None, 256, 128, None) == -1
    assert lib.pkv_dequant(ctypes.byref(c), P, 1, P, None, 1, P, P, 0, 128, None) == -1
    assert lib.pkv_dequant(ctypes.byref(c), None, 1, P, None, 1, P, P, 256, 128, None) == -1
    o = pkv._opts()
    dec = lambda *a: lib.pkv_decode_gqa(*a)
    # Hq not a multiple of Hkv
    assert dec(P, 3, ctypes.byref(c), P, 8, P, None, 1, 1, 1.0, P, None, P, 1 << 30, ctypes.byref(o), None) == -1
    # missing output
    assert dec(P, 4, ctypes.byref(c), P, 8, P, None, 1, 1, 1.0, None, None, P, 1 << 30, ctypes.byref(o), None) == -1
    # workspace too small for a split plan
    need = lib.pkv_decode_workspace_size(64, 32, 2, 128, 1024, 16, 1, 0, ctypes.byref(o))
    assert need > 0
    assert dec(P, 32, ctypes.byref(c), P, 1024, P, None, 64, 1, 1.0, P, None, P, need - 1,
               ctypes.byref(o), None) == -3
    assert dec(P, 32, ctypes.byref(c), P, 1024, P, None, 64, 1, 1.0, P, None, None, 0,
               ctypes.byref(o), None) == -3
    # reserved option fields must be zero
    o2 = pkv._opts()
    o2.reserved[1] = 1
    assert dec(P, 4, ctypes.byref(c), P, 8, P, None, 1, 1, 1.0, P, None, P, 1 << 30, ctypes.byref(o2), None) == -1
    o3 = pkv._opts(partition=3)  # no such partition
    assert dec(P, 4, ctypes.byref(c), P, 8, P, None, 1, 1, 1.0, P, None, P, 1 << 30, ctypes.byref(o3), None) == -1
    o4 = pkv._opts(window=-1)  # a window is a positive number of keys (0: none)
    assert dec(P, 4, ctypes.byref(c), P, 8, P, None, 1, 1, 1.0, P, None, P, 1 << 30, ctypes.byref(o4), None) == -1
    assert ctypes.sizeof(pkv._DecodeOpts) == 32  # split_tokens, kernel, partition, window, reserved[4]
    # unsupported head_dim
    bad = _cache_struct(pkv, hd=80)
    assert dec(P, 4, ctypes.byref(bad), P, 8, P, None, 1, 1, 1.0, P, None, P, 1 << 30, ctypes.byref(o), None) == -2
    # empty batch is a no-op
    assert dec(P, 4, ctypes.byref(c), P, 8, P, None, 0, 1, 1.0, P, None, None, 0, ctypes.byref(o), None) == 0


def test_sliding_window_plans_splits_over_the_window_only():
    """With a window the plan splits only the keys one row group can need (window + the chunk's
    spread + the 128-key alignment), not the whole block table."""
    import paged_kv_cache_c8_amd as pkv

    full = pkv.decode_plan(8, 64, 8, 128, 1024, 128, 1, 0, split_tokens=1024)
    win = pkv.decode_plan(8, 64, 8, 128, 1024, 128, 1, 0, split_tokens=1024, window=4096)
    assert full["num_splits"] == 128 and win["num_splits"] == 5  # ceil((4096 + 127) / 1024)


def test_mla_plan_and_argument_checks(pkv):
    lib = pkv.lib()
    P = 4096
    p = pkv.mla_decode_plan(64, 16, 128, 64)
    assert p == pkv.mla_decode_plan(64, 16, 128, 64)
    # the library's plan: a balanced partition over the GPU's resident workgroups (split length 0),
    # or, where the device is unknown, fixed splits covering the table
    assert (p["split_tokens"] == 0 and p["num_splits"] >= 128) or (
        p["split_tokens"] % 64 == 0 and p["num_splits"] * p["split_tokens"] >= 128 * 64)
    assert pkv.mla_decode_plan(64, 16, 128, 64, split_tokens=1000) == {"split_tokens": 1024, "num_splits": 8}
    assert pkv.mla_decode_plan(2, 16, 7, 16, split_tokens=100000)["num_splits"] == 1
    ws = pkv.mla_decode_workspace_size(64, 16, 128, 64, split_tokens=1024)
    # partials: (sequence, split) x 16 heads x (512 fp16 channels + fp32 lse and latent scale)
    assert ws == 64 * 8 * 16 * (512 * 2 + 2 * 4)
    assert pkv.mla_decode_workspace_size(64, 17, 128, 64, split_tokens=1024) == 2 * ws  # 2 head groups
    assert pkv.mla_decode_workspace_size(2, 16, 7, 16, split_tokens=100000) == 0
    c = pkv._MLACacheT(16, 32, 64, 128, 4, 16, 512, 64)
    st = lambda cache, *a: lib.pkv_mla_store_c8(ctypes.byref(cache), *a)
    assert st(c, P, P, 0, None, None, P, P, 1, 1, None) == 0    # nothing to do
    assert st(c, P, P, -1, None, None, P, P, 1, 1, None) == -1  # negative tokens
    assert st(c, P, P, 2, None, None, P, P, 1, 1, None) == -1   # decode form: T != B
    assert st(c, P + 8, P, 1, None, None, P, P, 1, 1, None) == -1  # latent rows not 16-byte aligned
    assert st(pkv._MLACacheT(16, 32, 64, 128, 4, 16, 256, 64), P, P, 1, None, None, P, P, 1, 1, None) == -2
    assert st(pkv._MLACacheT(16, 32, 64, 128, 4, 24, 512, 64), P, P, 1, None, None, P, P, 1, 1, None) == -2
    assert st(pkv._MLACacheT(16, 32, 0, 128, 4, 16, 512, 64), P, P, 1, None, None, P, P, 1, 1, None) == -1
    dec = lambda *a: lib.pkv_mla_decode(*a)
    assert dec(P, P, 16, ctypes.byref(c), P, 8, P, 1, 1.0, None, None, P, 1 << 30, 0, None) == -1  # no out
    assert dec(P, P, 0, ctypes.byref(c), P, 8, P, 1, 1.0, P, None, P, 1 << 30, 0, None) == -1  # no heads
    need = lib.pkv_mla_decode_workspace_size(64, 16, 128, 64, 0)
    assert need > 0
    c64 = pkv._MLACacheT(16, 32, 64, 128, 4, 64, 512, 64)
    assert dec(P, P, 16, ctypes.byref(c64), P, 128, P, 64, 1.0, P, None, P, need - 1, 0, None) == -3
    assert dec(P, P, 16, ctypes.byref(c64), P, 128, P, 0, 1.0, P, None, None, 0, 0, None) == 0  # empty batch
    walk = lambda cache, *a: lib.pkv_mla_cache_walk(ctypes.byref(cache), *a)
    assert walk(c64, P, 128, P, 0, 640, P, None) == 0       # empty batch: nothing launched
    assert walk(c64, P, 128, P, -1, 640, P, None) == -1     # negative batch
    assert walk(c64, P, 128, P, 1, 96, P, None) == -1       # split not a multiple of 64
    assert walk(c64, P, 128, P, 1, 8192, P, None) == -1     # split above 4096
    assert walk(c64, P, 128, P, 1, 640, P + 2, None) == -1  # out not 4-byte aligned
    assert walk(c64, None, 128, P, 1, 640, P, None) == -1   # no block table
    assert walk(pkv._MLACacheT(16, 32, 64, 128, 4, 64, 256, 64), P, 128, P, 1, 640, P, None) == -2


def test_check_indices_rejects_bad_arguments(pkv):
    """pkv_check_indices: argument errors are reported before anything is launched."""
    lib = pkv.lib()
    P = 4096
    chk = lambda *a: lib.pkv_check_indices(*a)
    #      num_blocks, bs, bt, mbs, ctx, cu, max_q, batch, slot, ntok, result, stream
    assert chk(8, 16, P, 4, P, None, 0, 2, None, 0, None, None) == -1  # no result
    assert chk(8, 16, P, 4, P, None, 0, 2, None, 0, P + 2, None) == -1  # misaligned result
    assert chk(8, 16, P, 4, None, None, 0, 2, None, 0, P, None) == -1  # block table without lengths
    assert chk(8, 16, P, 0, P, None, 0, 2, None, 0, P, None) == -1  # block table without a row size
    assert chk(8, 16, None, 0, None, None, 0, 2, None, 0, P, None) == -1  # nothing to check
    assert chk(8, 16, None, 0, None, None, 0, 0, None, 3, P, None) == -1  # tokens without slots
    assert chk(-1, 16, P, 4, P, None, 0, 2, None, 0, P, None) == -1
    assert chk(8, 0, P, 4, P, None, 0, 2, None, 0, P, None) == -1


def test_debug_environment_overrides(pkv, monkeypatch):
    """PKV_SPLIT_TOKENS and PKV_DECODE_PATH stand in for arguments left at 0, never for given ones."""
    base = pkv.decode_plan(8, 64, 8, 128, 1024, 128, 1, 0)
    monkeypatch.setenv("PKV_SPLIT_TOKENS", "1000")
    assert pkv.decode_plan(8, 64, 8, 128, 1024, 128, 1, 0)["split_tokens"] == 1024
    assert pkv.decode_plan(8, 64, 8, 128, 1024, 128, 1, 0, split_tokens=512)["split_tokens"] == 512
    monkeypatch.delenv("PKV_SPLIT_TOKENS")
    assert pkv.decode_plan(8, 64, 8, 128, 1024, 128, 1, 0) == base
    for path, kernel in (("valu", 1), ("mfma", 2), ("c8", 3)):
        monkeypatch.setenv("PKV_DECODE_PATH", path)
        assert pkv.decode_plan(2, 8, 2, 64, 7, 16, 1, 0)["kernel"] == kernel
    assert pkv.decode_plan(2, 8, 2, 64, 7, 16, 1, 0, kernel=2)["kernel"] == 2
    monkeypatch.setenv("PKV_DECODE_PATH", "cuda")
    with pytest.raises(ValueError):
        pkv.decode_plan(2, 8, 2, 64, 7, 16, 1, 0)
