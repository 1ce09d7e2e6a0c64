"""Attention as the pages define it, in float64 (test infrastructure only).

The definition (``attention``) materialises the whole score matrix, exactly
like the "standard attention" the [KVFA] HBM/SRAM section describes: scores
S = Q K^T, a softmax over each row, then P V.  We add the two things the
source pages state elsewhere: the 1/sqrt(d_head) score scale ([KPF], code in
"Following one new token through the cache", which divides by the square root
of the head size) and the causal mask (a query at absolute position p may see
keys 0..p).

The other functions restate the page's own algorithms so that tests can show
they reach the definition: the single-pass online softmax ([KVFA], online
softmax section; [KPF] worked example in "Flash attention: stop carrying
everything back and forth"), the tiled flash loop ([KVFA], Flash Attention
section) and the split-context merge of (m, l, O) partials, which is the same
rescale by exp(m_old - m_new) applied across splits instead of tiles
([KVFA], Flash Attention section; [DF], FlashAttention paragraphs).
"""
import math

import numpy as np


def softmax_rows(S):
    """Row softmax of a float64 matrix: exp(S - rowmax) / rowsum.

    Subtracting the row maximum before exponentiating is the standard guard
    against overflow that [KPF] mentions in its worked example; masked entries
    are -inf and contribute exp(-inf) = 0.
    """
    S = np.asarray(S, dtype=np.float64)
    mx = np.max(S, axis=-1, keepdims=True)
    E = np.exp(S - mx)
    return E / np.sum(E, axis=-1, keepdims=True)


def visible_keys(q_pos, L, window=0, sinks=0):
    """Boolean [Tq, L]: key j is visible to the query at position p iff
    j <= p (causal) and, when a window w > 0 is given, j is one of the w
    most recent positions p - w + 1 .. p or one of the first `sinks`
    positions.  The window is the sliding window of [KPF] "Sparse attention"
    (each token sees only the previous w tokens) and [KVFA] eviction
    paragraph (a window drops the oldest tokens); the sinks are the first
    few tokens that attention-sink eviction always keeps ([KVFA], same
    paragraph).  window = 0 means no window (full causal attention)."""
    j = np.arange(L)[None, :]
    p = np.asarray(q_pos)[:, None]
    vis = j <= p
    if window > 0:
        vis &= (j > p - window) | (j < sinks)
    return vis


def attention(q, k, v, scale, q_pos=None, window=0, sinks=0):
    """Causal softmax attention of one head, fully materialised, float64.

    q: [Tq, d] queries; k, v: [L, d] keys and values in logical order.
    q_pos: absolute position of each query row (default: the last Tq
    positions, i.e. L - Tq .. L - 1, which is the bottom-right alignment a
    decode step or a whole-prompt prefill both use).  Key j is visible to a
    query at position p iff j <= p, restricted by a sliding window and
    attention sinks when window > 0 (``visible_keys``).
    Returns O = softmax(q k^T * scale + mask) v, shape [Tq, d].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Tq, L = q.shape[0], k.shape[0]
    if q_pos is None:
        q_pos = np.arange(L - Tq, L)
    q_pos = np.asarray(q_pos)
    S = (q @ k.T) * scale
    visible = visible_keys(q_pos, L, window, sinks)
    S = np.where(visible, S, -np.inf)
    P = softmax_rows(S)
    return P @ v


def gqa_attention(q, k, v, scale, q_pos=None, window=0, sinks=0):
    """Grouped-query attention over all heads, float64.

    q: [Tq, n_q, d]; k, v: [L, n_kv, d] with n_q a multiple of n_kv.  Query
    head h reads key/value head h // (n_q / n_kv): the pages say only that
    several query heads share one key/value head ([KVFA] memory-cost section;
    [DF] architecture paragraph; [KPF] "Opening the hood"), and contiguous
    groups are the plain reading.  Returns [Tq, n_q, d].
    """
    q = np.asarray(q, dtype=np.float64)
    n_q, n_kv = q.shape[1], k.shape[1]
    assert n_q % n_kv == 0
    G = n_q // n_kv
    out = np.empty(q.shape, dtype=np.float64)
    for h in range(n_q):
        g = h // G
        out[:, h, :] = attention(q[:, h, :], k[:, g, :], v[:, g, :], scale, q_pos, window, sinks)
    return out


def tile_summary(block):
    """The softmax summary of one tile of scores on its own: its maximum m_t
    and l_t = sum over the tile of exp(x - m_t)."""
    m_t = max(block)
    return m_t, sum(math.exp(x - m_t) for x in block)


def combine_summaries(a, b):
    """Two (m, l) summaries of disjoint score sets -> the summary of their union.

    Both sums are brought to the common maximum M = max(m_a, m_b): a sum taken
    against m is multiplied by exp(m - M), the correction [KVFA] (online
    softmax section) and [DF] (running-summary paragraph) apply whenever the
    running maximum rises.  The empty summary (-inf, 0) is the identity: its
    factor is taken as 0, since exp(-inf - M) is 0.
    """
    (m_a, l_a), (m_b, l_b) = a, b
    M = max(m_a, m_b)
    if M == -math.inf:
        return M, 0.0
    f_a = 0.0 if m_a == -math.inf else math.exp(m_a - M)
    f_b = 0.0 if m_b == -math.inf else math.exp(m_b - M)
    return M, l_a * f_a + l_b * f_b


def online_softmax_trace(scores, tile):
    """Single pass over a row of scores in tiles, keeping (m, l).

    The running state starts as the empty summary (-inf, 0); each tile's own
    summary is folded into it with ``combine_summaries``, so after tile t the
    state is the (max, sum of exp(x - max)) of every score seen so far,
    without the earlier scores being revisited ([KVFA] online softmax
    section; [DF] running-summary paragraph; [KPF] worked example in "Flash
    attention").  Returns the state after each tile.
    """
    state = (-math.inf, 0.0)
    trace = []
    for t0 in range(0, len(scores), tile):
        state = combine_summaries(state, tile_summary([float(x) for x in scores[t0:t0 + tile]]))
        trace.append(state)
    return trace


def online_softmax(scores, tile):
    """Probabilities from the single-pass (m, l): exp(x - m) / l."""
    m, l = online_softmax_trace(scores, tile)[-1]
    return np.array([math.exp(float(x) - m) / l for x in scores])


def flash_attention_tiled(q, k, v, scale, tile_q, tile_k, q_pos=None):
    """The page's tiled flash loop for one head, with scale and causal mask.

    Outer loop over query tiles, inner loop over key/value tiles; each query
    row carries (m, l, O) and every new tile rescales l and O by
    exp(m_old - m_new) before adding its own contribution; one division by l
    at the end of the row tile ([KVFA], Flash Attention section).  A masked
    score is -inf; a row whose tile is fully masked so far keeps m = -inf and
    its rescale factor is taken as 0, the guard the online softmax section
    uses.  Float64 throughout.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Tq, d = q.shape
    L = k.shape[0]
    if q_pos is None:
        q_pos = np.arange(L - Tq, L)
    q_pos = np.asarray(q_pos)
    O = np.zeros((Tq, v.shape[1]))
    for i in range(0, Tq, tile_q):
        Qi = q[i:i + tile_q]
        pos_i = q_pos[i:i + tile_q]
        m_i = np.full(Qi.shape[0], -np.inf)
        l_i = np.zeros(Qi.shape[0])
        O_i = np.zeros((Qi.shape[0], v.shape[1]))
        for j in range(0, L, tile_k):
            Kj, Vj = k[j:j + tile_k], v[j:j + tile_k]
            S = (Qi @ Kj.T) * scale
            cols = np.arange(j, j + Kj.shape[0])
            S = np.where(cols[None, :] <= pos_i[:, None], S, -np.inf)
            m_new = np.maximum(m_i, S.max(axis=1))
            live = m_new > -np.inf
            safe_m = np.where(live, m_new, 0.0)
            P = np.where(live[:, None], np.exp(S - safe_m[:, None]), 0.0)
            alpha = np.where(m_i > -np.inf, np.exp(m_i - safe_m), 0.0)
            l_i = alpha * l_i + P.sum(axis=1)
            O_i = alpha[:, None] * O_i + P @ Vj
            m_i = m_new
        O[i:i + tile_q] = O_i / l_i[:, None]
    return O


def split_partials(q, k, v, scale, split_len):
    """Per-split (m, l, O) of one decode query row over its whole context.

    q: [d]; k, v: [L, d].  Split s covers keys [s*split_len, (s+1)*split_len).
    For each split: m_s = max of its scores, l_s = sum exp(score - m_s) and
    O_s = sum exp(score - m_s) v (unnormalised), i.e. the running state the
    online softmax holds after sweeping that split alone.
    Returns arrays m [S], l [S], O [S, d].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    L = k.shape[0]
    n_split = -(-L // split_len)
    ms, ls, Os = [], [], []
    for s in range(n_split):
        sl = slice(s * split_len, min((s + 1) * split_len, L))
        sc = (k[sl] @ q) * scale
        m_s = sc.max()
        p = np.exp(sc - m_s)
        ms.append(m_s)
        ls.append(p.sum())
        Os.append(p @ v[sl])
    return np.array(ms), np.array(ls), np.array(Os)


def merge_partials(m, l, O):
    """Merge split partials: M = max m_s, w_s = exp(m_s - M),
    result = sum_s w_s O_s / sum_s w_s l_s.

    Each split's state is brought to the common maximum by the same
    exp(m_old - m_new) rescale the online softmax applies tile by tile.
    """
    m = np.asarray(m, dtype=np.float64)
    M = m.max()
    w = np.exp(m - M)
    return (w[:, None] * np.asarray(O)).sum(axis=0) / (w * np.asarray(l)).sum()


def decode_attention(q, k, v, scale, window=0, sinks=0):
    """One decode step of one sequence: every cached row is visible.

    q: [n_q, d] (the new token's queries), k, v: [L, n_kv, d] with the new
    token's own row already appended (the cache appends before the query
    attends, [KPF] "Following one new token through the cache").
    Returns [n_q, d].
    """
    q = np.asarray(q, dtype=np.float64)
    return gqa_attention(q[None], k, v, scale, q_pos=[k.shape[0] - 1], window=window,
                         sinks=sinks)[0]


def prefill_attention(q, k, v, scale, window=0, sinks=0):
    """Causal attention of a whole prompt on an empty cache.

    q: [T, n_q, d]; k, v: [T, n_kv, d]; query t sees keys 0..t.
    Returns [T, n_q, d].
    """
    T = np.asarray(q).shape[0]
    return gqa_attention(q, k, v, scale, q_pos=np.arange(T), window=window, sinks=sinks)


def extend_attention(q, k, v, scale, window=0, sinks=0):
    """k new query rows against a cache that already holds their own rows.

    The cache holds L rows (the k new tokens' K/V rows included, appended
    before the queries attend); the queries are the last k positions
    L - k .. L - 1, and query t sees keys 0 .. L - k + t.  This is one chunk
    of a prompt processed against the cache the earlier chunks filled
    ([KVFA] continuous-batching section: chunked prefill folded into a decode
    iteration; [KPF] prefill spikes split into chunks), and it is the target
    model's single pass over k drafted positions ([KVFA] speculative-decoding
    section).
    q: [k, n_q, d]; k, v: [L, n_kv, d] with L >= k.  Returns [k, n_q, d].
    """
    Tq, L = np.asarray(q).shape[0], np.asarray(k).shape[0]
    assert 1 <= Tq <= L
    return gqa_attention(q, k, v, scale, q_pos=np.arange(L - Tq, L), window=window, sinks=sinks)
