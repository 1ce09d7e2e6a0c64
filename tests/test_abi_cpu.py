"""The C ABI on the CPU: exported symbols, closed forms, the host allocator
(through a host-only handle) against the oracle's paged model, and error
codes.  No device call is made."""
import ctypes
import os
import random
import re

import pytest

import pins
import kv_cache_flashattention_amd as kv
from oracle.paged import PagedCacheModel

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "include", "kvfa.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kvc_\w+)\s*\(", src)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert len(names) >= 17
    L = kv.lib()
    for n in names:
        assert hasattr(L, n), n
        assert n in kv._SIGS, f"binding does not marshal {n}"


def test_bytes_per_token_through_the_abi():
    for case in pins.golden("closed_forms.json")["bytes_per_token"]:
        dt = {2: "bf16", 1: "fp8", 4: "f32"}[case["bytes"]]
        cfg = kv.make_config(case["n_layers"], case["n_kv_heads"], case["n_kv_heads"],
                             case["d_head"], 16, 1, 1, dt)
        assert kv.bytes_per_token(cfg) == case["expected"], case["source"]
    fp8 = kv.make_config(80, 64, 8, 128, 16, 1, 1, "fp8")
    f16 = kv.make_config(80, 64, 8, 128, 16, 1, 1, "f16")
    assert kv.bytes_per_token(f16) == 2 * kv.bytes_per_token(fp8)
    i4 = kv.make_config(80, 64, 8, 128, 16, 1, 1, "int4")
    assert kv.bytes_per_token(fp8) == 2 * kv.bytes_per_token(i4) == 80 * 8 * 128 * 2


def test_required_sizes():
    cfg = kv.make_config(2, 8, 2, 64, 10, 3, 5, "fp8")
    s = kv.required_sizes(cfg)
    assert s["k_pool"] == s["v_pool"] == 2 * 10 * 2 * 16 * 64
    assert s["k_scale"] == s["v_scale"] == 2 * 10 * 2 * 4
    assert s["block_table"] == 3 * 5 * 4 and s["seq_len"] == 3 * 4
    s = kv.required_sizes(kv.make_config(1, 4, 4, 128, 7, 2, 2, "bf16"))
    assert s["k_pool"] == 7 * 4 * 16 * 128 * 2 and s["k_scale"] == 0
    s = kv.required_sizes(kv.make_config(2, 8, 2, 64, 10, 3, 5, "int4"))
    assert s["k_pool"] == s["v_pool"] == 2 * 10 * 2 * 16 * 64 // 2
    assert s["k_scale"] == s["v_scale"] == 2 * 10 * 2 * 4


def test_unknown_dtype_rejected():
    cfg = kv.make_config(1, 8, 2, 64, 4, 2, 4, "int4")
    cfg.kv_dtype = 5
    with pytest.raises(kv.KvcError) as e:
        kv.required_sizes(cfg)
    assert e.value.code == kv.KVC_E_INVAL


@pytest.mark.parametrize("bad", [dict(d_head=96), dict(n_q_heads=6, n_kv_heads=4),
                                 dict(block=8)])
def test_unsupported_configs(bad):
    args = dict(n_layers=1, n_q_heads=8, n_kv_heads=2, d_head=64, n_blocks=4, max_seqs=2,
                max_blocks_per_seq=4, kv_dtype="bf16")
    block = bad.pop("block", 16)
    args.update(bad)
    cfg = kv.make_config(**args)
    cfg.block_size = block
    with pytest.raises(kv.KvcError) as e:
        kv.required_sizes(cfg)
    assert e.value.code == kv.KVC_E_UNSUPPORTED


def host_cache(n_blocks=40, max_seqs=6, max_bps=8):
    return kv.KvCache(1, 4, 2, 64, n_blocks, max_seqs, max_bps, "bf16", device=None)


def assert_same(c, m):
    assert c.free_blocks() == len(m.free)
    assert [c.block_refs(b) for b in range(len(m.refs))] == m.refs
    for s in range(c.cfg.max_seqs):
        if s in m.table:
            assert c.seq_blocks(s) == m.table[s] and c.seq_len(s) == m.length[s]
        else:
            with pytest.raises(kv.KvcError):
                c.seq_len(s)


def test_allocator_matches_the_page_listing_model():
    rng = random.Random(0)
    c, m = host_cache(), PagedCacheModel(1, 2, 64, "bf16", 40, 6, 8, poison=False)
    for step in range(400):
        op = rng.random()
        live = sorted(m.table)
        if op < 0.3:
            s = rng.randrange(6)
            n = rng.randrange(0, 60)
            try:
                m.alloc(s, n) if s not in m.table else (_ for _ in ()).throw(KeyError())
                ok = True
            except (MemoryError, KeyError):
                ok = False
            if ok:
                c.seq_alloc(s, n)
            else:
                with pytest.raises(kv.KvcError):
                    c.seq_alloc(s, n)
        elif op < 0.38 and live:
            src = rng.choice(live)
            free_ids = [x for x in range(6) if x not in m.table]
            if not free_ids:
                continue
            dst = rng.choice(free_ids)
            plen = rng.randrange(0, m.length[src] + 1)
            m.share_prefix(src, dst, plen)
            c.seq_share_prefix(src, dst, plen)
        elif op < 0.45 and live:
            s = rng.choice(live)
            n = rng.randrange(0, 40)
            need = -(-(m.length[s] + n) // 16) - -(-m.length[s] // 16)
            need += 1 if n > 0 and m._shared_partial(s) else 0
            if m.length[s] + n > 8 * 16:
                with pytest.raises(kv.KvcError) as e:
                    c.seq_grow_by(s, n)
                assert e.value.code == kv.KVC_E_INVAL
            elif need > len(m.free):
                with pytest.raises(kv.KvcError) as e:
                    c.seq_grow_by(s, n)
                assert e.value.code == kv.KVC_E_NO_BLOCKS
            else:
                m.grow_by(s, n)
                c.seq_grow_by(s, n)
        elif op < 0.8 and live:
            seqs = rng.sample(live, rng.randrange(1, len(live) + 1))
            if any(m.length[s] + 1 > 8 * 16 for s in seqs):
                continue
            need = sum(1 for s in seqs if m.length[s] % 16 == 0 or m._shared_partial(s))
            if need > len(m.free):
                with pytest.raises(kv.KvcError) as e:
                    c.seq_grow(seqs)
                assert e.value.code == kv.KVC_E_NO_BLOCKS
            else:
                m.grow(seqs)
                c.seq_grow(seqs)
        elif live:
            s = rng.choice(live)
            m.release(s)
            c.seq_release(s)
        assert_same(c, m)
        held = [b for t in m.table.values() for b in t]
        assert not set(held) & set(m.free)
        assert all(m.refs[b] == held.count(b) for b in set(held))


def test_exhaustion_leaves_state_unchanged():
    c = host_cache(n_blocks=3)
    c.seq_alloc(0, 16)
    c.seq_alloc(1, 32)
    assert c.free_blocks() == 0
    before = (c.seq_blocks(0), c.seq_len(0), c.seq_blocks(1), c.seq_len(1))
    with pytest.raises(kv.KvcError) as e:
        c.seq_grow([1, 0])                    # both need a block
    assert e.value.code == kv.KVC_E_NO_BLOCKS
    assert (c.seq_blocks(0), c.seq_len(0), c.seq_blocks(1), c.seq_len(1)) == before
    with pytest.raises(kv.KvcError) as e:
        c.seq_alloc(2, 1)
    assert e.value.code == kv.KVC_E_NO_BLOCKS
    c.seq_release(1)
    assert c.free_blocks() == 2
    c.seq_grow([0])
    assert c.seq_len(0) == 17 and c.seq_blocks(0) == [2, 0]   # release pushed [1, 0]; pop takes 0


def test_error_codes():
    c = host_cache()
    c.seq_alloc(0, 5)
    cases = [
        (lambda: c.seq_alloc(0, 1), kv.KVC_E_STATE),          # already live
        (lambda: c.seq_alloc(9, 1), kv.KVC_E_INVAL),          # id out of range
        (lambda: c.seq_alloc(1, 8 * 16 + 1), kv.KVC_E_INVAL),  # wider than the table
        (lambda: c.seq_grow([0, 0]), kv.KVC_E_INVAL),         # duplicate
        (lambda: c.seq_grow([1]), kv.KVC_E_STATE),            # not live
        (lambda: c.seq_release(3), kv.KVC_E_STATE),
    ]
    for fn, code in cases:
        with pytest.raises(kv.KvcError) as e:
            fn()
        assert e.value.code == code
    c.set_block_table(1, [0, 1], 17)
    with pytest.raises(kv.KvcError) as e:
        c.set_block_table(2, [1], 3)                          # block 1 is owned
    assert e.value.code == kv.KVC_E_STATE
    with pytest.raises(kv.KvcError) as e:
        c.set_block_table(2, [3, 4], 3)                       # nblk != ceil(len/16)
    assert e.value.code == kv.KVC_E_INVAL
    assert kv.lib().kvc_last_error().decode() != ""


def test_host_only_handle_refuses_device_calls():
    c = host_cache()
    c.seq_alloc(0, 4)
    L = kv.lib()
    rc = L.kvc_append(c._h, 0, 1, ctypes.c_void_p(16), ctypes.c_void_p(16),
                      ctypes.c_void_p(16), None)
    assert rc == kv.KVC_E_STATE
    rc = L.kvc_attn_decode(c._h, 0, 1, ctypes.c_void_p(16), ctypes.c_void_p(16),
                           ctypes.c_void_p(16), ctypes.c_float(1.0), 0, None, 0, None)
    assert rc == kv.KVC_E_STATE
    rc = L.kvc_attn_decode_noalloc(c._h, 0, 1, ctypes.c_void_p(16), ctypes.c_void_p(16),
                                   ctypes.c_void_p(16), ctypes.c_float(1.0), 0, None)
    assert rc == kv.KVC_E_STATE
    # grow + append in one launch: refused before any bookkeeping changes
    ids = (ctypes.c_int32 * 1)(0)
    rc = L.kvc_seq_grow_append(c._h, 0, 1, ids, ctypes.c_void_p(16), ctypes.c_void_p(16), None)
    assert rc == kv.KVC_E_STATE
    assert c.seq_len(0) == 4


@pytest.mark.parametrize("scale", [0.0, -0.125, float("nan"), float("inf")])
def test_attention_rejects_scale_outside_positive_reals(scale):
    """Both attention calls take the row max on unscaled scores, which is only
    the max of the scaled scores for a positive multiplier."""
    c = host_cache()
    L = kv.lib()
    p = ctypes.c_void_p(16)
    rc = L.kvc_attn_decode(c._h, 0, 1, p, p, p, ctypes.c_float(scale), 0, None, 0, None)
    assert rc == kv.KVC_E_INVAL
    rc = L.kvc_attn_prefill(c._h, 0, 1, None, 4, p, p, p, p, ctypes.c_float(scale), None)
    assert rc == kv.KVC_E_INVAL


def test_decode_workspace_plan():
    """Matrix-core caches use a work list: (sequence x group segments + waves)
    slots of 16 rows x (d + 2) floats plus the batch's prefix sums; f32 caches
    use fixed splits per (sequence, query head)."""
    c = kv.KvCache(1, 32, 8, 128, 6000, 64, 300, "bf16", device=None)
    assert c.decode_workspace_bytes(40) == 0               # nothing live yet
    c.seq_alloc(0, 4096)
    assert c.decode_workspace_bytes(40) > 0
    segs, waves = 40 * 8, 40 * 8 * 4
    want = (segs + waves) * 16 * 130 * 4 + 41 * 8 + 40 * 4 + 16
    assert c.decode_workspace_bytes(40, num_splits=4) == want
    f = kv.KvCache(1, 32, 8, 128, 6000, 64, 300, "f32", device=None)
    f.seq_alloc(0, 4096)
    assert f.decode_workspace_bytes(40, num_splits=1) == 0
    assert f.decode_workspace_bytes(40, num_splits=4) == 40 * 32 * 4 * 130 * 4


@pytest.mark.parametrize("dtype", ["f32"])
def test_extend_refuses_cache_types_without_a_kernel(dtype):
    c = kv.KvCache(1, 8, 2, 128, 16, 2, 4, dtype, device=None)
    p = ctypes.c_void_p(16)
    rc = kv.lib().kvc_attn_extend(c._h, 0, 1, p, 4, p, p, ctypes.c_float(0.1), None)
    assert rc == kv.KVC_E_UNSUPPORTED


def test_window_arguments_are_checked():
    p = ctypes.c_void_p(16)
    L = kv.lib()
    c = kv.KvCache(1, 8, 2, 128, 16, 2, 4, "bf16", device=None)
    rc = L.kvc_attn_decode_window(c._h, 0, 1, p, p, p, ctypes.c_float(0.1), -1, 0, 0, None, 0,
                                  None)
    assert rc == kv.KVC_E_INVAL
    rc = L.kvc_attn_prefill_window(c._h, 0, 1, None, 4, p, p, p, p, ctypes.c_float(0.1), 8, -2,
                                   None)
    assert rc == kv.KVC_E_INVAL
    rc = L.kvc_attn_extend_window(c._h, 0, 1, p, 4, p, p, ctypes.c_float(0.1), -3, 0, None)
    assert rc == kv.KVC_E_INVAL
    f = kv.KvCache(1, 8, 2, 128, 16, 2, 4, "f32", device=None)
    rc = L.kvc_attn_decode_window(f._h, 0, 1, p, p, p, ctypes.c_float(0.1), 8, 0, 0, None, 0, None)
    assert rc == kv.KVC_E_UNSUPPORTED
    rc = L.kvc_attn_prefill_window(f._h, 0, 1, None, 4, p, p, p, p, ctypes.c_float(0.1), 8, 0,
                                   None)
    assert rc == kv.KVC_E_UNSUPPORTED


def test_share_prefix_and_copy_on_write_bookkeeping():
    """Sharing a prefix that ends inside a block: both sequences hold it
    (refcount 2); the first grow of either one moves it to a fresh block
    and leaves the other one alone; releases free a block only when its
    last holder goes."""
    c, m = host_cache(), PagedCacheModel(1, 2, 64, "bf16", 40, 6, 8, poison=False)
    for x in (c, m):
        (x.seq_alloc if x is c else x.alloc)(0, 40)               # blocks for rows 0..39
    c.seq_share_prefix(0, 1, 36)
    m.share_prefix(0, 1, 36)
    assert_same(c, m)
    shared = c.seq_blocks(0)
    assert c.seq_blocks(1) == shared and all(c.block_refs(b) == 2 for b in shared)
    c.seq_grow([1])                                                # row 36 of seq 1: copy
    m.grow([1])
    assert_same(c, m)
    assert c.seq_blocks(1)[:2] == shared[:2] and c.seq_blocks(1)[2] != shared[2]
    assert c.block_refs(shared[2]) == 1
    c.seq_grow([0])                                                # row 40 of seq 0: no copy
    m.grow([0])
    assert_same(c, m) and c.seq_blocks(0) == shared
    c.seq_share_prefix(1, 2, 32)                                   # whole blocks: no copy later
    m.share_prefix(1, 2, 32)
    c.seq_grow_by(2, 5)
    m.grow_by(2, 5)
    assert_same(c, m)
    assert c.seq_blocks(2)[:2] == shared[:2]
    free0 = c.free_blocks()
    c.seq_release(0)
    m.release(0)
    assert_same(c, m)
    assert c.free_blocks() == free0 + 1                            # only block 2 of seq 0
    with pytest.raises(kv.KvcError) as e:
        c.seq_share_prefix(1, 2, 3)                                # dst already live
    assert e.value.code == kv.KVC_E_STATE
    with pytest.raises(kv.KvcError) as e:
        c.seq_share_prefix(1, 3, 38)                               # longer than src
    assert e.value.code == kv.KVC_E_INVAL
