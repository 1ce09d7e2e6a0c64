"""Checks that pin the oracle to facts outside itself.

Each check takes the oracle function(s) it examines as arguments and returns
True when the function agrees with what the source pages print, a closed
form, an invariant, a library routine or brute force.  test_oracle_pins.py
runs them against the real oracle; test_oracle_mutations.py runs them
against deliberately broken copies to show that each pin catches a plausible
mistake.
"""
import json
import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def r3(x):
    return round(float(x), 3)


# ------------------------------------------------------------ online softmax
def check_worked_example(trace_fn):
    """The printed worked example: tiles [1,2] then [3,0]."""
    g = golden("online_softmax_worked_example.json")
    tr = trace_fn(g["scores"], g["tile"])
    (m1, l1), (m2, l2) = tr
    ok = m1 == g["after_tile_1"]["m"] and r3(l1) == g["after_tile_1"]["l"]
    ok &= r3(math.exp(m1 - m2)) == g["tile_2"]["rescale_factor"]
    ok &= r3(l1 * math.exp(m1 - m2)) == g["tile_2"]["rescaled_l"]
    ok &= m2 == g["final"]["m"] and r3(l2) == g["final"]["l"]
    direct = sum(math.exp(x - max(g["scores"])) for x in g["scores"])
    ok &= r3(direct) == g["direct_sum_against_max_3"]
    ok &= abs(l2 - direct) <= 1e-15 * direct
    return bool(ok)


def check_online_every_split(online_fn, seed=0):
    """Tiled single-pass probabilities equal the direct softmax for every
    tile width of random rows (float64, relative 1e-14)."""
    rng = np.random.default_rng(seed)
    for n in (1, 2, 3, 7, 16, 33):
        x = rng.standard_normal(n) * 5
        ref = np.exp(x - x.max()) / np.exp(x - x.max()).sum()
        for tile in range(1, n + 1):
            p = online_fn(list(x), tile)
            if not np.allclose(p, ref, rtol=1e-14, atol=0):
                return False
    return True


# ------------------------------------------------------------ attention
def sdpa_ref(q, k, v, scale, causal):
    """torch's scaled_dot_product_attention on the CPU in float64.
    q [Tq, n_q, d], k/v [L, n_kv, d] -> [Tq, n_q, d]."""
    Q = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2)))[None].double()
    K = torch.from_numpy(np.ascontiguousarray(k.transpose(1, 0, 2)))[None].double()
    V = torch.from_numpy(np.ascontiguousarray(v.transpose(1, 0, 2)))[None].double()
    out = torch.nn.functional.scaled_dot_product_attention(
        Q, K, V, is_causal=causal, scale=scale, enable_gqa=True)
    return out[0].numpy().transpose(1, 0, 2)


def check_prefill_vs_sdpa(prefill_fn, seed=1):
    """Whole-prompt causal attention equals torch SDPA (is_causal, T == L)."""
    rng = np.random.default_rng(seed)
    for (T, n_q, n_kv, d) in ((1, 4, 2, 8), (37, 8, 2, 16), (64, 6, 6, 32), (19, 8, 1, 16)):
        q = rng.standard_normal((T, n_q, d))
        k = rng.standard_normal((T, n_kv, d))
        v = rng.standard_normal((T, n_kv, d))
        scale = 1 / math.sqrt(d)
        if not np.allclose(prefill_fn(q, k, v, scale), sdpa_ref(q, k, v, scale, True),
                           rtol=0, atol=1e-12):
            return False
    return True


def check_decode_vs_sdpa(decode_fn, seed=2):
    """One decode row sees the whole cache: torch SDPA without a mask."""
    rng = np.random.default_rng(seed)
    for (L, n_q, n_kv, d) in ((1, 4, 2, 8), (50, 8, 2, 16), (129, 4, 4, 32), (33, 16, 1, 8)):
        q = rng.standard_normal((n_q, d))
        k = rng.standard_normal((L, n_kv, d))
        v = rng.standard_normal((L, n_kv, d))
        scale = 1 / math.sqrt(d)
        ref = sdpa_ref(q[None], k, v, scale, False)[0]
        if not np.allclose(decode_fn(q, k, v, scale), ref, rtol=0, atol=1e-12):
            return False
    return True


def sdpa_masked_ref(q, k, v, scale, q_pos):
    """torch SDPA in float64 with an explicit boolean mask: key j visible to
    the query at position p iff j <= p.  q [Tq, n_q, d], k/v [L, n_kv, d]."""
    L = k.shape[0]
    Q = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2)))[None].double()
    K = torch.from_numpy(np.ascontiguousarray(k.transpose(1, 0, 2)))[None].double()
    V = torch.from_numpy(np.ascontiguousarray(v.transpose(1, 0, 2)))[None].double()
    mask = torch.from_numpy(np.arange(L)[None, :] <= np.asarray(q_pos)[:, None])
    out = torch.nn.functional.scaled_dot_product_attention(
        Q, K, V, attn_mask=mask, scale=scale, enable_gqa=True)
    return out[0].numpy().transpose(1, 0, 2)


def check_extend_vs_sdpa(extend_fn, seed=11):
    """k query rows at positions L-k..L-1 against L cached rows equal torch
    SDPA with the explicit bottom-right mask."""
    rng = np.random.default_rng(seed)
    for (k_, L, n_q, n_kv, d) in ((1, 1, 4, 2, 8), (3, 40, 8, 2, 16), (17, 17, 4, 4, 8),
                                  (5, 70, 16, 1, 8), (33, 100, 6, 3, 16)):
        q = rng.standard_normal((k_, n_q, d))
        kc = rng.standard_normal((L, n_kv, d))
        vc = rng.standard_normal((L, n_kv, d))
        scale = 1 / math.sqrt(d)
        ref = sdpa_masked_ref(q, kc, vc, scale, np.arange(L - k_, L))
        if not np.allclose(extend_fn(q, kc, vc, scale), ref, rtol=0, atol=1e-12):
            return False
    return True


def check_chunked_equals_whole(extend_fn, prefill_fn, seed=12):
    """Chunked prefill: a prompt processed in consecutive chunks, each chunk's
    queries against the cache filled up to the chunk's end, gives the rows of
    the whole-prompt causal prefill.  Also k = 1 against L rows is one decode
    row and k = L is the whole prompt."""
    rng = np.random.default_rng(seed)
    T, n_q, n_kv, d = 45, 8, 2, 16
    q = rng.standard_normal((T, n_q, d))
    kc = rng.standard_normal((T, n_kv, d))
    vc = rng.standard_normal((T, n_kv, d))
    scale = 1 / math.sqrt(d)
    whole = prefill_fn(q, kc, vc, scale)
    for cuts in ((0, 10, 11, 30, 45), (0, 1, 2, 3, 45), (0, 45)):
        for a, b in zip(cuts[:-1], cuts[1:]):
            got = extend_fn(q[a:b], kc[:b], vc[:b], scale)
            if not np.allclose(got, whole[a:b], rtol=0, atol=1e-12):
                return False
    return True


def check_window_vs_sdpa(attention_fn, seed=13):
    """Window/sink masks: equal torch SDPA with the explicit boolean mask
    built from the rule written out element by element."""
    rng = np.random.default_rng(seed)
    for (Tq, L, w, s, d) in ((1, 50, 8, 0, 8), (1, 50, 8, 3, 8), (20, 20, 5, 2, 16),
                             (7, 90, 30, 4, 8), (33, 100, 1, 0, 8), (33, 100, 1, 5, 8),
                             (10, 40, 64, 2, 8)):
        q = rng.standard_normal((Tq, 2, d))
        k = rng.standard_normal((L, 1, d))
        v = rng.standard_normal((L, 1, d))
        pos = np.arange(L - Tq, L)
        mask = np.zeros((Tq, L), dtype=bool)
        for i, p in enumerate(pos):
            for j in range(L):
                mask[i, j] = j <= p and (p - j < w or j < s)
        Q = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2)))[None].double()
        K = torch.from_numpy(np.ascontiguousarray(k.transpose(1, 0, 2)))[None].double()
        V = torch.from_numpy(np.ascontiguousarray(v.transpose(1, 0, 2)))[None].double()
        ref = torch.nn.functional.scaled_dot_product_attention(
            Q, K, V, attn_mask=torch.from_numpy(mask), scale=1 / math.sqrt(d),
            enable_gqa=True)[0].numpy().transpose(1, 0, 2)
        got = attention_fn(q, k, v, 1 / math.sqrt(d), pos, w, s)
        if not np.allclose(got, ref, rtol=0, atol=1e-12):
            return False
    return True


def check_window_special_cases(attention_fn, seed=14):
    """A window of 1 without sinks returns each query's own value row; a
    window at least as long as the context is full causal attention; a
    window with sinks equals full attention over the kept rows gathered
    explicitly (sinks, then the window), for one decode row."""
    rng = np.random.default_rng(seed)
    L, d = 60, 8
    q = rng.standard_normal((L, 1, d))
    k = rng.standard_normal((L, 1, d))
    v = rng.standard_normal((L, 1, d))
    pos = np.arange(L)
    if not np.array_equal(attention_fn(q, k, v, 0.3, pos, 1, 0)[:, 0], v[:, 0]):
        return False
    if not np.allclose(attention_fn(q, k, v, 0.3, pos, L, 0),
                       attention_fn(q, k, v, 0.3, pos, 0, 0), rtol=0, atol=1e-14):
        return False
    w, s = 12, 4
    keep = np.r_[0:s, L - w:L]
    got = attention_fn(q[-1:], k, v, 0.3, [L - 1], w, s)
    sc = (k[keep, 0] @ q[-1, 0]) * 0.3
    e = np.exp(sc - sc.max())
    ref = (e / e.sum()) @ v[keep, 0]
    return bool(np.allclose(got[0, 0], ref, rtol=0, atol=1e-13))


def check_tiled_equals_definition(tiled_fn, attention_fn, seed=3):
    """The tiled flash loop (any tile sizes) reaches the definition."""
    rng = np.random.default_rng(seed)
    for (Tq, L, d) in ((37, 37, 8), (1, 45, 8), (5, 70, 16)):
        q = rng.standard_normal((Tq, d))
        k = rng.standard_normal((L, d))
        v = rng.standard_normal((L, d))
        ref = attention_fn(q, k, v, 0.3)
        for tq in (1, 3, 16, 64, Tq):
            for tk in (1, 3, 16, 64, L):
                if not np.allclose(tiled_fn(q, k, v, 0.3, tq, tk), ref, rtol=0, atol=1e-12):
                    return False
    return True


def check_merge_equals_definition(partials_fn, merge_fn, attention_fn, seed=4):
    """Split partials merged by the (m, l) rule equal one-pass decode."""
    rng = np.random.default_rng(seed)
    for L in (1, 15, 16, 17, 100, 257):
        q = rng.standard_normal(16)
        k = rng.standard_normal((L, 16)) * 2
        v = rng.standard_normal((L, 16))
        ref = attention_fn(q[None], k, v, 0.25)[0]
        for split in (1, 2, 16, 64, 256, 1000):
            m, l, O = partials_fn(q, k, v, 0.25, split)
            if not np.allclose(merge_fn(m, l, O), ref, rtol=0, atol=1e-12):
                return False
    return True


def cache_demo(attention_fn, d=16, n=6, seed=0):
    """The one-head demo: outputs and K/V row counts with and without a cache.

    Projections W ~ N(0,1)/sqrt(d); without a cache every step recomputes the
    K/V of the whole prefix; with one, only the new token's row is computed
    and appended before its query attends."""
    rng = np.random.Generator(np.random.PCG64(seed))
    Wq, Wk, Wv = (rng.standard_normal((d, d)) / math.sqrt(d) for _ in range(3))
    x = rng.standard_normal((n, d))
    scale = 1 / math.sqrt(d)
    outs_no, rows_no = [], 0
    for t in range(1, n + 1):
        K, V = x[:t] @ Wk, x[:t] @ Wv
        rows_no += t
        full = attention_fn(x[:t] @ Wq, K, V, scale)       # all t query rows, causal
        outs_no.append(full[-1])                           # keep only the last row
    Kc, Vc, outs_c = [], [], []
    for t in range(1, n + 1):
        new = x[t - 1]
        Kc.append(new @ Wk)
        Vc.append(new @ Wv)
        outs_c.append(attention_fn((new @ Wq)[None], np.array(Kc), np.array(Vc), scale)[0])
    return np.array(outs_no), np.array(outs_c), rows_no, len(Kc)


def check_cache_demo(attention_fn):
    g = golden("cache_demo.json")
    a, b, rows_no, rows_c = cache_demo(attention_fn, g["d"], g["tokens"])
    same = bool(np.allclose(a, b, rtol=0, atol=1e-12))
    return same == g["same_outputs"] and rows_no == g["rows_without_cache"] \
        and rows_c == g["rows_with_cache"]


def check_invariants(attention_fn, seed=5):
    rng = np.random.default_rng(seed)
    d = 8
    for L in (1, 2, 9, 40):
        q = rng.standard_normal((1, d))
        k = rng.standard_normal((L, d))
        v = rng.standard_normal((L, d))
        o = attention_fn(q, k, v, 0.5)[0]
        if np.any(o < v.min(axis=0) - 1e-12) or np.any(o > v.max(axis=0) + 1e-12):
            return False                                   # convex combination of rows
        if L == 1 and not np.array_equal(o, v[0]):
            return False                                   # a single row is returned exactly
        keq = np.repeat(k[:1], L, axis=0)
        if not np.allclose(attention_fn(q, keq, v, 0.5)[0], v.mean(axis=0), atol=1e-12):
            return False                                   # equal keys: uniform weights
        # weights sum to one: attending over V = all-ones gives exactly ones
        if not np.allclose(attention_fn(q, k, np.ones((L, 3)), 0.5), 1.0, atol=1e-14):
            return False
    return True


def check_gqa_is_repeated_mha(gqa_fn, seed=6):
    """GQA equals MHA with each kv head repeated G times in contiguous groups."""
    rng = np.random.default_rng(seed)
    T, n_q, n_kv, d = 11, 12, 3, 8
    q = rng.standard_normal((T, n_q, d))
    k = rng.standard_normal((T, n_kv, d))
    v = rng.standard_normal((T, n_kv, d))
    G = n_q // n_kv
    kr, vr = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)
    pos = np.arange(T)
    return bool(np.allclose(gqa_fn(q, k, v, 0.3, pos), gqa_fn(q, kr, vr, 0.3, pos),
                            rtol=0, atol=0))


# ------------------------------------------------------------ codecs
def _brute_e4m3(x, table):
    """Nearest finite code by exhaustive search; ties go to the even code;
    magnitudes beyond 448 saturate."""
    finite = [(c, table[c]) for c in range(256) if not math.isnan(table[c])]
    out = []
    for val in np.asarray(x, dtype=np.float64).ravel():
        a = min(abs(val), 448.0)
        pos = [(c, t) for c, t in finite if t >= 0 and not (t == 0 and c == 0x80)]
        best = min(pos, key=lambda ct: (abs(ct[1] - a), ct[0] & 1))
        code = best[0]
        if math.copysign(1.0, val) < 0:
            code |= 0x80
        out.append(code)
    return np.array(out, dtype=np.uint8)


def fp8_probe_values(table, n_random=3000, seed=7):
    """Float32 values at and around every rounding boundary plus random ones."""
    pos = sorted(set(float(t) for t in table if not math.isnan(t) and t >= 0))
    vals = []
    for a, b in zip(pos[:-1], pos[1:]):
        mid = np.float32((a + b) / 2)
        vals += [a, b, mid, np.nextafter(mid, np.float32(0)), np.nextafter(mid, np.float32(1e9))]
    vals += [448.0, 449.0, 464.0, 465.0, 1e6, 2.0 ** -12, 2.0 ** -10, 0.0]
    rng = np.random.default_rng(seed)
    vals += list(rng.standard_normal(n_random).astype(np.float32) * 30)
    vals += list((rng.random(n_random) * 2.0 ** -6).astype(np.float32))
    v = np.array(vals, dtype=np.float32)
    return np.concatenate([v, -v])


def check_e4m3_table(table):
    finite = table[~np.isnan(table)]
    return bool(len(finite) == 254 and np.nanmax(table) == 448.0
                and np.isnan(table[0x7F]) and np.isnan(table[0xFF])
                and table[1] == 2.0 ** -9 and table[0x08] == 2.0 ** -6
                and table[0x38] == 1.0 and table[0x7E] == 448.0 and table[0xFE] == -448.0
                and len(set(finite.tolist())) == 253)          # +0 and -0 compare equal


def check_e4m3_encode_brute(encode_fn, table):
    x = fp8_probe_values(table)
    return bool(np.array_equal(encode_fn(x), _brute_e4m3(x, table)))


def check_e4m3_encode_torch(encode_fn, table):
    """Within +-448 the encoder equals torch's float8_e4m3fn cast (which rounds
    to nearest even but does not saturate, so larger values are left out)."""
    x = fp8_probe_values(table)
    x = x[np.abs(x) <= 448.0]
    t = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return bool(np.array_equal(encode_fn(x), t))


def check_e4m3_roundtrip(encode_fn, table):
    codes = np.array([c for c in range(256) if not math.isnan(table[c])], dtype=np.uint8)
    return bool(np.array_equal(encode_fn(table[codes]), codes))


def check_bf16_vs_torch(bits_fn, seed=8):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000)).astype(np.float32)
    ties = (np.arange(1, 2000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, -ties, np.float32([0.0, -0.0, 3.0e38, 1e-40])])
    t = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return bool(np.array_equal(bits_fn(x), t))


def check_int4_encode_brute(encode_fn, seed=15):
    """Nearest of the 15 levels -7..7 by brute force, ties to the even level,
    saturation beyond +-7, for random values and every tie point."""
    rng = np.random.default_rng(seed)
    ys = np.concatenate([rng.uniform(-9, 9, 4000).astype(np.float32),
                         np.arange(-8.5, 8.6, 0.5, dtype=np.float32),
                         np.array([-0.0, 0.0, 7.49, -7.51, 100.0, -1e6], dtype=np.float32)])
    levels = np.arange(-7, 8)
    got = encode_fn(ys)
    for y, c in zip(ys.astype(np.float64), got):
        dist = np.abs(levels - y)
        best = levels[dist == dist.min()]
        want = best[0] if len(best) == 1 else best[best % 2 == 0][0]
        if int(c) != int(want):
            return False
    return True


def check_int4_slab_rule(slab_fn, seed=16):
    """After every write the scale is absmax/7 of all rows written; decoded
    values stay within (k+1)/2 scale steps after k re-encodings; rows above
    the written ones keep their codes."""
    rng = np.random.default_rng(seed)
    d = 8
    codes = np.full((16, d), 5, dtype=np.int8)
    scale, r0, seen = np.float32(0), 0, []
    for n in (3, 1, 5, 2, 4):
        rows = (rng.standard_normal((n, d)) * rng.uniform(0.1, 10)).astype(np.float32)
        codes, scale = slab_fn(codes, scale, r0, rows)
        seen.append(rows)
        allr = np.concatenate(seen)
        if np.float32(scale) != np.float32(np.abs(allr).max() / np.float32(7)):
            return False
        if not np.all(codes[r0 + n:] == 5):
            return False
        k = len(seen)
        err = np.abs(codes[:r0 + n].astype(np.float64) * scale - allr)
        if np.any(err > (k + 1) / 2 * scale * (1 + 1e-6)):
            return False
        r0 += n
    return True
