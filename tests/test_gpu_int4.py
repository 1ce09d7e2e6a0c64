"""int4 caches on the GPU: codes and scales byte for byte against the
oracle's paged model (bulk writes, kv_append with requantisation, mid-block
writes, the gather), and decode against the oracle on the dequantised values
the cache holds.  Parity against the unquantised rows is not claimed: the
pages fix no int4 format."""
import math

import numpy as np
import pytest
import torch

import kv_cache_flashattention_amd as kv
from harness import Built, assert_close, bits, f64, pools_match, stored_rows
from oracle import attention as A
from oracle.paged import PagedCacheModel
from workloads import DecodeWorkload, decode_workload

pytestmark = pytest.mark.gpu


def _q(w, io=torch.bfloat16):
    return torch.from_numpy(w.q()).to(io).cuda()


@pytest.mark.parametrize("d", [64, 128])
def test_int4_write_append_pools_bit_exact(d):
    w = DecodeWorkload("i4cache", 5, 8, 2, d, "int4", (1, 70), outliers=True)
    b = Built(w, n_layers=2, layer=1)
    assert b.pools_equal()


def test_int4_append_requantises_growing_block():
    """Rows appended one at a time with growing magnitudes: every code, both
    nibbles of every byte, and every scale follow the slab rule."""
    c = kv.KvCache(1, 4, 1, 128, 4, 1, 4, "int4", poison=True)
    m = PagedCacheModel(1, 1, 128, "int4", 4, 1, 4, poison=True)
    c.seq_alloc(0, 0)
    m.alloc(0, 0)
    seqs = torch.zeros(1, dtype=torch.int32, device="cuda")
    rng = np.random.default_rng(0)
    for r in range(40):
        mag = [0.0, 1e-3, 1.0, 0.5, 7.0, 3.0, 300.0, 1e4][r % 8] * (1 + r // 8)
        row = (rng.standard_normal((1, 1, 128)) * mag).astype(np.float32)
        k = torch.from_numpy(row).to(torch.bfloat16).cuda()
        v = torch.from_numpy(row[:, :, ::-1].copy()).to(torch.bfloat16).cuda()
        c.seq_grow([0])
        m.grow([0])
        c.append(0, seqs, k.contiguous(), v.contiguous())
        m.write_rows(0, 0, r, k.float().cpu().numpy(), v.float().cpu().numpy())
        torch.cuda.synchronize()
        assert pools_match(c, m), f"row {r}"


def test_int4_write_mid_block_matches_slab_rule():
    """Bulk writes that start and stop inside blocks (odd and even rows, so
    both nibbles of V bytes change separately), on top of earlier rows."""
    c = kv.KvCache(1, 8, 2, 64, 12, 2, 8, "int4", poison=True)
    m = PagedCacheModel(1, 2, 64, "int4", 12, 2, 8, poison=True)
    c.set_block_table(0, [7, 2, 9, 4], 60)
    m.set_table(0, [7, 2, 9, 4], 60)
    seqs = torch.zeros(1, dtype=torch.int32, device="cuda")
    rng = np.random.default_rng(1)
    for start, T, mag in ((0, 5, 1.0), (5, 20, 3.0), (25, 3, 0.1), (28, 1, 9.0), (29, 31, 50.0)):
        rows = (rng.standard_normal((1, T, 2, 64)) * mag).astype(np.float32)
        k = torch.from_numpy(rows).to(torch.bfloat16).cuda()
        v = torch.from_numpy(-rows).to(torch.bfloat16).cuda()
        c.write(0, seqs, start, k, v)
        m.write_rows(0, 0, start, k[0].float().cpu().numpy(), v[0].float().cpu().numpy())
        torch.cuda.synchronize()
        assert pools_match(c, m), f"write at {start}"


def test_int4_gather_returns_packed_logical_rows():
    w = DecodeWorkload("i4gather", 4, 8, 2, 128, "int4", (20, 90))
    b = Built(w)
    for s in range(w.batch):
        L = int(w.lengths[s])
        for start, count in ((0, L), (L // 3, L - L // 3), (L - 1, 1)):
            k, v = b.c.gather(0, s, start, count)
            mk, mv = stored_rows(b.m, 0, s, start, count)
            assert np.array_equal(bits(k), mk) and np.array_equal(bits(v), mv)


@pytest.mark.parametrize("splits", [0, 1, 3])
def test_int4_decode_small_workload(splits):
    w = decode_workload("llama70b_decode_int4", small=True)
    b = Built(w)
    q = _q(w)
    y = f64(b.c.attn_decode(0, b.seqs, q, num_splits=splits))
    assert_close(y, b.oracle_decode(q), what=f"int4 splits={splits}")


@pytest.mark.parametrize("n_q,n_kv,d,lengths", [(20, 4, 64, (1, 200)), (32, 1, 128, (1, 200)),
                                                (8, 8, 128, (1, 40)), (40, 8, 64, (300, 700))])
def test_int4_decode_shapes(n_q, n_kv, d, lengths):
    w = DecodeWorkload(f"i4shape{n_q}-{n_kv}-{d}", 4, n_q, n_kv, d, "int4", lengths,
                       outliers=True)
    b = Built(w)
    q = _q(w)
    for splits in (0, 2, 7):
        y = f64(b.c.attn_decode(0, b.seqs, q, num_splits=splits))
        assert_close(y, b.oracle_decode(q), what=f"int4 {n_q}/{n_kv}/{d} splits={splits}")


def test_int4_decode_reproduces_every_code_exactly():
    """A one-row cache whose row holds every code -7..7 (absmax 7, scale 1):
    decode returns the row itself, so the widening of codes (and the removal
    of the operands' offset) is exact for all 15 codes."""
    vals = np.tile(np.arange(-7, 8, dtype=np.float32), 18)[:256]
    row = vals.reshape(1, 2, 128)
    c = kv.KvCache(1, 2, 2, 128, 2, 1, 2, "int4", poison=True)
    c.seq_alloc(0, 0)
    c.seq_grow([0])
    seqs = torch.zeros(1, dtype=torch.int32, device="cuda")
    k = torch.from_numpy(row).to(torch.bfloat16).cuda()
    c.append(0, seqs, k, k)
    q = torch.ones(1, 2, 128, dtype=torch.bfloat16, device="cuda")
    y = c.attn_decode(0, seqs, q).float().cpu().numpy()
    assert np.array_equal(y.reshape(-1), vals), "decoded int4 values differ"
    assert float(c.v_scale[0, c.seq_blocks(0)[0], 0]) == 1.0


def test_int4_scores_use_every_code():
    """Two rows whose keys differ in one dimension by each code step: the
    attention weights (hence the output) follow the oracle on the stored
    values, so K's widening is exact too."""
    rng = np.random.default_rng(5)
    c = kv.KvCache(1, 1, 1, 64, 2, 1, 2, "int4", poison=True)
    m = PagedCacheModel(1, 1, 64, "int4", 2, 1, 2, poison=True)
    c.seq_alloc(0, 16)
    m.alloc(0, 16)
    k = np.tile(np.arange(-7, 8, dtype=np.float32), 70)[:16 * 64].reshape(1, 16, 1, 64)
    k = k * rng.choice([-1.0, 1.0], size=k.shape).astype(np.float32)
    k[0, 0, 0, 0] = 7.0
    v = rng.standard_normal((1, 16, 1, 64)).astype(np.float32)
    kt = torch.from_numpy(k).to(torch.bfloat16).cuda()
    vt = torch.from_numpy(v).to(torch.bfloat16).cuda()
    seqs = torch.zeros(1, dtype=torch.int32, device="cuda")
    c.write(0, seqs, 0, kt, vt)
    m.write_rows(0, 0, 0, kt[0].float().cpu().numpy(), vt[0].float().cpu().numpy())
    for trial in range(4):
        q = torch.from_numpy(rng.standard_normal((1, 1, 64)).astype(np.float32) * 2).to(
            torch.bfloat16).cuda()
        y = f64(c.attn_decode(0, seqs, q))
        K, V = m.logical_values(0, 0)
        r = A.decode_attention(f64(q[0]), K, V, 1 / math.sqrt(64))
        assert_close(y[0], r, what=f"trial {trial}")


def test_int4_decode_window_and_sinks():
    w = decode_workload("llama70b_decode_int4", small=True)
    b = Built(w)
    q = _q(w)
    scale = 1 / math.sqrt(w.d)
    for window, sinks in ((64, 0), (100, 4), (17, 33)):
        y = f64(b.c.attn_decode(0, b.seqs, q, window=window, sinks=sinks))
        for s in range(w.batch):
            K, V = b.m.logical_values(0, s)
            r = A.decode_attention(f64(q[s]), K, V, scale, window=window, sinks=sinks)
            assert_close(y[s], r, what=f"int4 decode w={window} s={sinks} seq {s}")


@pytest.mark.parametrize("dtype", ["int4", "fp8"])
def test_prefill_with_scaled_cache_writes_codes_and_attends_in_bf16(dtype):
    """Prefill on an fp8 / int4 cache: attention runs on the bf16 inputs
    (oracle tolerance), and the cache holds exactly the codes and scales of
    the oracle's slab rule applied to the prompt rows, after which decode
    against the cache matches the oracle on the dequantised values."""
    from workloads import prefill_workload
    w = prefill_workload(small=True)
    qn, kn, vn = w.qkv()
    q, k, v = (torch.from_numpy(a).to(torch.bfloat16).cuda() for a in (qn, kn, vn))
    nb = -(-w.T // 16)
    c = kv.KvCache(1, w.n_q, w.n_kv, w.d, w.batch * nb + 3, w.batch, nb + 1, dtype, poison=True)
    m = PagedCacheModel(1, w.n_kv, w.d, dtype, w.batch * nb + 3, w.batch, nb + 1, poison=True)
    for s in range(w.batch):
        c.seq_alloc(s, w.T)
        m.alloc(s, w.T)
    seqs = torch.arange(w.batch, dtype=torch.int32, device="cuda")
    out = c.attn_prefill(0, q, k, v, seqs=seqs)
    torch.cuda.synchronize()
    scale = 1 / math.sqrt(w.d)
    for s in range(w.batch):
        ref = A.prefill_attention(f64(q[s]), f64(k[s]), f64(v[s]), scale)
        assert_close(f64(out[s]), ref, what=f"prefill seq {s}")
        m.write_rows(0, s, 0, k[s].float().cpu().numpy(), v[s].float().cpu().numpy())
    assert pools_match(c, m)
    qd = q[:, -1].contiguous()                            # decode the last prompt row again
    y = f64(c.attn_decode(0, seqs, qd))
    for s in range(w.batch):
        K, V = m.logical_values(0, s)
        assert_close(y[s], A.decode_attention(f64(qd[s]), K, V, scale), what=f"decode seq {s}")


@pytest.mark.parametrize("splits", [0, 1, 3])
@pytest.mark.parametrize("which", ["k", "v"])
@pytest.mark.parametrize("dtype", ["fp8", "int4"])
def test_decode_nan_block_scale_gives_nan_rows(dtype, which, splits):
    """The scale arrays are caller memory: a NaN K or V scale in one (block,
    kv head) makes exactly the query rows of that sequence and kv head NaN
    (their softmax or weighted sum cannot be evaluated), and every other row
    still matches the oracle -- under the work list, where the poisoned unit
    may be the only one of its piece, and under fixed split counts."""
    n_q, n_kv, d = 8, 2, 128
    w = DecodeWorkload("nanscale" + dtype, 3, n_q, n_kv, d, dtype, 300)
    b = Built(w)
    q = torch.from_numpy(w.q()).to(b.io).cuda()
    blk = b.c.seq_blocks(1)[2]
    (b.c.k_scale if which == "k" else b.c.v_scale)[0, blk, 0] = float("nan")
    torch.cuda.synchronize()
    y = f64(b.c.attn_decode(0, b.seqs, q, num_splits=splits))
    G = n_q // n_kv
    assert np.all(np.isnan(y[1, :G])), "rows of the poisoned (sequence, kv head)"
    scale = 1 / math.sqrt(d)
    for s in range(w.batch):
        K, V = b.m.logical_values(0, s)
        r = A.decode_attention(f64(q[s]), K, V, scale)
        rows = slice(G, n_q) if s == 1 else slice(0, n_q)
        assert_close(y[s, rows], r[rows], what=f"{dtype} sequence {s}")
