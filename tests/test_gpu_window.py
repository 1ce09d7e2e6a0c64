"""GPU parity of the sliding-window / attention-sink variants of decode,
prefill and extend against the float64 oracle with the same mask (key j
visible to position p iff j <= p and (p - window < j or j < sinks))."""
import math

import numpy as np
import pytest
import torch

import kv_cache_flashattention_amd as kv
from harness import FP8_ABS_TOL, Built, assert_close, f64
from oracle import attention as A
from workloads import decode_workload

pytestmark = pytest.mark.gpu

CASES = [(1, 0), (5, 0), (31, 2), (32, 0), (33, 1), (100, 4), (100, 40), (300, 7), (2000, 3)]


def _rows(rng, shape, io):
    return torch.from_numpy(rng.standard_normal(shape, dtype=np.float32)).to(io).cuda()


def _cache(dtype, n_q, n_kv, d, lengths, seed):
    rng = np.random.default_rng(seed)
    io = kv.IO_TORCH[dtype]
    nbs = [-(-L // 16) for L in lengths]
    n_blocks = sum(nbs) + 3
    c = kv.KvCache(1, n_q, n_kv, d, n_blocks, len(lengths), max(nbs) + 1, dtype, poison=True)
    perm = rng.permutation(n_blocks).astype(np.int32)
    o, rows = 0, []
    for b, L in enumerate(lengths):
        c.set_block_table(b, perm[o:o + nbs[b]], L)
        o += nbs[b]
        k, v = _rows(rng, (1, L, n_kv, d), io), _rows(rng, (1, L, n_kv, d), io)
        c.write(0, torch.tensor([b], dtype=torch.int32, device="cuda"), 0, k, v)
        rows.append((k[0], v[0]))
    return c, rows


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f16", 64)])
def test_decode_window_vs_oracle(dtype, d):
    n_q, n_kv = 8, 2
    lengths = [1, 17, 64, 65, 250, 999, 1500]
    c, rows = _cache(dtype, n_q, n_kv, d, lengths, seed=d)
    rng = np.random.default_rng(1)
    q = _rows(rng, (len(lengths), n_q, d), kv.IO_TORCH[dtype])
    seqs = torch.arange(len(lengths), dtype=torch.int32, device="cuda")
    scale = 1 / math.sqrt(d)
    for window, sinks in CASES:
        out = c.attn_decode(0, seqs, q, window=window, sinks=sinks)
        torch.cuda.synchronize()
        for b, (k, v) in enumerate(rows):
            ref = A.decode_attention(f64(q[b]), f64(k), f64(v), scale, window, sinks)
            assert_close(f64(out[b]), ref, io=dtype,
                         what=f"decode {dtype} L={lengths[b]} w={window} s={sinks}")


def test_decode_window_fp8_vs_dequantised_oracle():
    w = decode_workload("llama70b_decode_fp8", small=True)
    B = Built(w)
    rng = np.random.default_rng(2)
    q = _rows(rng, (w.batch, w.n_q, w.d), torch.bfloat16)
    scale = 1 / math.sqrt(w.d)
    for window, sinks in ((40, 0), (100, 5), (513, 16)):
        out = B.c.attn_decode(0, B.seqs, q, window=window, sinks=sinks)
        torch.cuda.synchronize()
        for b in range(w.batch):
            K, V = B.m.logical_values(0, b)
            ref = A.decode_attention(f64(q[b]), K, V, scale, window, sinks)
            assert_close(f64(out[b]), ref, abs_tol=FP8_ABS_TOL,
                         what=f"fp8 decode w={window} s={sinks} seq {b}")


@pytest.mark.parametrize("dtype,d,T", [("bf16", 128, 300), ("f16", 64, 131), ("bf16", 64, 700)])
def test_prefill_window_vs_oracle(dtype, d, T):
    n_q, n_kv = 8, 2
    rng = np.random.default_rng(T)
    io = kv.IO_TORCH[dtype]
    q, k, v = (_rows(rng, (2, T, h, d), io) for h in (n_q, n_kv, n_kv))
    c = kv.KvCache(1, n_q, n_kv, d, 4, 1, 4, dtype)
    scale = 1 / math.sqrt(d)
    for window, sinks in CASES:
        out = c.attn_prefill(0, q, k, v, window=window, sinks=sinks)
        torch.cuda.synchronize()
        for s in range(2):
            ref = A.prefill_attention(f64(q[s]), f64(k[s]), f64(v[s]), scale, window, sinks)
            assert_close(f64(out[s]), ref, io=dtype,
                         what=f"prefill {dtype} T={T} w={window} s={sinks}")


def test_extend_window_vs_oracle():
    dtype, n_q, n_kv, d, T = "bf16", 8, 2, 128, 77
    lengths = [77, 200, 1100]
    c, rows = _cache(dtype, n_q, n_kv, d, lengths, seed=9)
    rng = np.random.default_rng(10)
    q = _rows(rng, (len(lengths), T, n_q, d), kv.IO_TORCH[dtype])
    seqs = torch.arange(len(lengths), dtype=torch.int32, device="cuda")
    scale = 1 / math.sqrt(d)
    for window, sinks in CASES:
        out = c.attn_extend(0, seqs, q, window=window, sinks=sinks)
        torch.cuda.synchronize()
        for b, (k, v) in enumerate(rows):
            ref = A.extend_attention(f64(q[b]), f64(k), f64(v), scale, window, sinks)
            assert_close(f64(out[b]), ref, what=f"extend L={lengths[b]} w={window} s={sinks}")
