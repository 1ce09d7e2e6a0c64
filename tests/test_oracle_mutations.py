"""Plant plausible mistakes in copies of oracle functions (on the CPU) and
show that the pins reject every one of them."""
import math

import numpy as np

import pins
from oracle import attention as A
from oracle import codecs as C


def _fold(scores, tile, combine):
    """online_softmax_trace with a planted combine rule."""
    state, tr = (-math.inf, 0.0), []
    for t0 in range(0, len(scores), tile):
        state = combine(state, A.tile_summary([float(x) for x in scores[t0:t0 + tile]]))
        tr.append(state)
    return tr


def test_online_softmax_without_rescale_is_caught():
    def no_rescale(a, b):                              # sums added without the exp factors
        return max(a[0], b[0]), a[1] + b[1]
    assert not pins.check_worked_example(lambda s, t: _fold(s, t, no_rescale))


def test_online_softmax_wrong_sign_is_caught():
    def wrong_sign(a, b):                              # exp(M - m) instead of exp(m - M)
        M = max(a[0], b[0])
        fa = math.exp(M - a[0]) if a[0] != -math.inf else 0.0
        fb = math.exp(M - b[0]) if b[0] != -math.inf else 0.0
        return M, a[1] * fa + b[1] * fb
    assert not pins.check_worked_example(lambda s, t: _fold(s, t, wrong_sign))

    def online(scores, tile):
        m, l = _fold(scores, tile, wrong_sign)[-1]
        return np.array([math.exp(x - m) / l for x in scores])
    assert not pins.check_online_every_split(online)


def test_online_softmax_stale_maximum_is_caught():
    def stale_max(a, b):                               # keeps the first tile's maximum
        if a[0] == -math.inf:
            return b
        return a[0], a[1] + b[1] * math.exp(b[0] - a[0])
    assert not pins.check_worked_example(lambda s, t: _fold(s, t, stale_max))


def test_missing_scale_is_caught():
    def no_scale(q, k, v, scale):
        return A.prefill_attention(q, k, v, 1.0)
    assert not pins.check_prefill_vs_sdpa(no_scale)


def test_top_left_causal_alignment_is_caught():
    def top_left(q, k, v, scale, q_pos=None):
        return A.attention(q, k, v, scale, q_pos=np.arange(np.asarray(q).shape[0]))
    assert not pins.check_cache_demo(top_left)

    def dec(q, k, v, scale):
        return A.gqa_attention(np.asarray(q)[None], k, v, scale, q_pos=[0])[0]
    assert not pins.check_decode_vs_sdpa(dec)


def test_strict_causal_mask_is_caught():
    def strict(q, k, v, scale, q_pos=None):
        q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
        Tq, L = q.shape[0], k.shape[0]
        pos = np.arange(L - Tq, L)
        S = (q @ k.T) * scale
        vis = np.arange(L)[None, :] < pos[:, None]       # the diagonal hidden
        vis[:, 0] = True
        S = np.where(vis, S, -np.inf)
        return A.softmax_rows(S) @ v
    assert not pins.check_invariants(strict) or not pins.check_cache_demo(strict)


def test_wrong_gqa_mapping_is_caught():
    def interleaved(q, k, v, scale, q_pos=None):
        n_q, n_kv = q.shape[1], k.shape[1]
        out = np.empty(q.shape)
        for h in range(n_q):
            g = h % n_kv                                  # round-robin instead of groups
            out[:, h] = A.attention(q[:, h], k[:, g], v[:, g], scale, q_pos)
        return out
    assert not pins.check_gqa_is_repeated_mha(interleaved)

    def prefill(q, k, v, scale):
        return interleaved(q, k, v, scale, np.arange(q.shape[0]))
    assert not pins.check_prefill_vs_sdpa(prefill)


def test_transposed_pv_is_caught():
    def transposed(q, k, v, scale, q_pos=None):
        q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
        Tq, L = q.shape[0], k.shape[0]
        pos = np.arange(L - Tq, L) if q_pos is None else np.asarray(q_pos)
        S = np.where(np.arange(L)[None] <= pos[:, None], (q @ k.T) * scale, -np.inf)
        P = A.softmax_rows(S)
        return (P @ v[::-1])                              # values in the wrong order
    def prefill(q, k, v, scale):
        out = np.empty(q.shape)
        G = q.shape[1] // k.shape[1]
        for h in range(q.shape[1]):
            out[:, h] = transposed(q[:, h], k[:, h // G], v[:, h // G], scale, np.arange(q.shape[0]))
        return out
    assert not pins.check_prefill_vs_sdpa(prefill)
    assert not pins.check_tiled_equals_definition(A.flash_attention_tiled, transposed)


def test_merge_without_weights_is_caught():
    def unweighted(m, l, O):
        return np.asarray(O).sum(axis=0) / np.asarray(l).sum()
    assert not pins.check_merge_equals_definition(A.split_partials, unweighted, A.attention)


def test_fp8_truncation_is_caught():
    def truncating(x):
        x = np.asarray(x, dtype=np.float64)
        sign = np.where(np.signbit(x), 0x80, 0)
        a = np.abs(x)
        _, E = np.frexp(a)
        e = np.where(a < 2.0 ** -6, -6, E - 1)
        n = np.floor(a / np.exp2(e - 3))                  # truncates instead of rounding
        code = np.where(a < 2.0 ** -6, n, ((e + 7) << 3) + n - 8)
        code = np.where(a >= 448, 0x7E, np.minimum(code, 0x7E))
        return (sign | code.astype(np.int64)).astype(np.uint8)
    assert not pins.check_e4m3_encode_brute(truncating, C.E4M3_TABLE)


def test_fp8_ties_away_is_caught():
    def ties_away(x):
        x = np.asarray(x, dtype=np.float64)
        sign = np.where(np.signbit(x), 0x80, 0)
        a = np.abs(x)
        _, E = np.frexp(a)
        e = np.where(a < 2.0 ** -6, -6, E - 1)
        n = np.floor(a / np.exp2(e - 3) + 0.5)            # ties away from zero
        code = np.where(a < 2.0 ** -6, n, ((e + 7) << 3) + n - 8)
        code = np.where(a >= 448, 0x7E, np.minimum(code, 0x7E))
        return (sign | code.astype(np.int64)).astype(np.uint8)
    assert not pins.check_e4m3_encode_brute(ties_away, C.E4M3_TABLE)
    assert not pins.check_e4m3_encode_torch(ties_away, C.E4M3_TABLE)


def test_fp8_wrong_bias_is_caught():
    bad = C.E4M3_TABLE * 2.0                              # exponent bias off by one
    assert not pins.check_e4m3_table(bad)


def test_bf16_truncation_is_caught():
    def trunc(x):
        return (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)
    assert not pins.check_bf16_vs_torch(trunc)


def test_fp8_slab_without_requant_is_caught():
    """A slab rule that raises the scale but leaves older codes alone decodes
    the older rows at the wrong scale; the error bound rejects it."""
    from test_oracle_pins import _slab_error_ok

    def no_requant(codes, scale, r0, new_rows):
        codes = np.array(codes, dtype=np.uint8, copy=True)
        new_rows = np.asarray(new_rows, dtype=np.float32)
        s_new = np.float32(np.float32(np.abs(new_rows).max()) / np.float32(448))
        s = s_new if r0 == 0 else np.float32(max(np.float32(scale), s_new))
        for i in range(new_rows.shape[0]):
            codes[r0 + i] = C.e4m3_encode((new_rows[i] / s).astype(np.float32))
        return codes, s

    rows = np.array([[1.0, -0.5], [4.0, 2.0]], dtype=np.float32)
    codes, s = no_requant(np.zeros((16, 2), np.uint8), np.float32(0), 0, rows[:1])
    codes, s = no_requant(codes, s, 1, rows[1:])
    assert not _slab_error_ok(codes, s, rows.astype(np.float64), 1)
    codes, s = C.fp8_slab_write(np.zeros((16, 2), np.uint8), np.float32(0), 0, rows[:1])
    codes, s = C.fp8_slab_write(codes, s, 1, rows[1:])
    assert _slab_error_ok(codes, s, rows.astype(np.float64), 1)


def test_extend_with_top_left_positions_is_caught():
    """Chunk queries placed at positions 0..k-1 instead of L-k..L-1."""
    def top_left(q, k, v, scale):
        return A.gqa_attention(q, k, v, scale, q_pos=np.arange(np.asarray(q).shape[0]))
    assert not pins.check_extend_vs_sdpa(top_left)
    assert not pins.check_chunked_equals_whole(top_left, A.prefill_attention)


def test_extend_off_by_one_is_caught():
    """Query t seeing keys 0..L-k+t-1 (its own row hidden)."""
    def strict(q, k, v, scale):
        Tq, L = np.asarray(q).shape[0], np.asarray(k).shape[0]
        return A.gqa_attention(q, k, v, scale, q_pos=np.arange(L - Tq, L) - 0.5)
    assert not pins.check_extend_vs_sdpa(strict)
    assert not pins.check_chunked_equals_whole(strict, A.prefill_attention)


def test_window_off_by_one_is_caught():
    """A window that keeps w + 1 rows (j >= p - w instead of j > p - w)."""
    def wide(q, k, v, scale, q_pos=None, window=0, sinks=0):
        return A.gqa_attention(q, k, v, scale, q_pos, window + 1 if window else 0, sinks)
    assert not pins.check_window_vs_sdpa(wide)
    assert not pins.check_window_special_cases(wide)


def test_sinks_ignored_is_caught():
    def no_sinks(q, k, v, scale, q_pos=None, window=0, sinks=0):
        return A.gqa_attention(q, k, v, scale, q_pos, window, 0)
    assert not pins.check_window_vs_sdpa(no_sinks)
    assert not pins.check_window_special_cases(no_sinks)


def test_int4_ties_away_is_caught():
    def ties_away(y):
        y = np.asarray(y, dtype=np.float64)
        return np.clip(np.sign(y) * np.floor(np.abs(y) + 0.5), -7, 7).astype(np.int8)
    assert not pins.check_int4_encode_brute(ties_away)


def test_int4_truncation_is_caught():
    def trunc(y):
        return np.clip(np.trunc(np.asarray(y, dtype=np.float64)), -7, 7).astype(np.int8)
    assert not pins.check_int4_encode_brute(trunc)


def test_int4_slab_without_requantisation_is_caught():
    def no_requant(codes, scale, r0, new_rows):
        codes = np.array(codes, dtype=np.int8, copy=True)
        new_rows = np.asarray(new_rows, dtype=np.float32)
        s_new = np.float32(np.abs(new_rows).max() / np.float32(7))
        s = s_new if r0 == 0 else np.float32(max(np.float32(scale), s_new))
        for i, row in enumerate(new_rows):
            codes[r0 + i] = C.int4_encode((row / s).astype(np.float32) if s > 0 else row)
        return codes, s
    assert not pins.check_int4_slab_rule(no_requant)
