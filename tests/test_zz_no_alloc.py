"""kvc_attn_decode_noalloc -- decode whose split partials live in the
library's own device scratch instead of a caller workspace -- against
kvc_attn_decode with a caller workspace, through the C ABI.  Both run the
same kernels with the same plan, so the outputs must be bit-identical; both
are also held to the oracle's tolerances.  Two calls in a row, the second
with fewer sequences and other queries, so that a stale entry left in the
shared scratch by the first call would show."""
import ctypes

import numpy as np
import pytest
import torch

import kv_cache_flashattention_amd as kv
from harness import Built, assert_close, f64
from workloads import DecodeWorkload, decode_workload

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.detach().view(torch.int16 if t.element_size() == 2 else torch.int32).cpu()


def _check_pair(b, seqs, q, num_splits=0):
    ref = b.c.attn_decode(0, seqs, q, num_splits=num_splits).clone()
    y = b.c.attn_decode_noalloc(0, seqs, q, num_splits=num_splits).clone()
    torch.cuda.synchronize()
    assert torch.equal(_bits(y), _bits(ref)), "no-alloc decode differs from the workspace decode"
    return y


@pytest.mark.parametrize("name", ["llama8b_decode", "llama70b_decode_fp8", "long_mha_decode",
                                  "llama70b_decode_int4"])
def test_noalloc_equals_workspace_decode_twice(name):
    w = decode_workload(name, small=True)
    b = Built(w)
    q = torch.from_numpy(w.q()).to(b.io).cuda()
    y1 = _check_pair(b, b.seqs, q)
    assert_close(f64(y1), b.oracle_decode(q), what=f"{name} first call", io=b.io_name)
    # second call: the last half of the batch, other queries
    n2 = max(1, w.batch // 2)
    seqs2 = b.seqs[w.batch - n2:].contiguous()
    q2 = (q[w.batch - n2:].float() * -0.75).to(b.io).contiguous()
    y2 = _check_pair(b, seqs2, q2)
    qfull = q.clone()
    qfull[w.batch - n2:] = q2
    ref2 = np.array([b.oracle_decode(qfull, s)[0] for s in range(w.batch - n2, w.batch)])
    assert_close(f64(y2), ref2, what=f"{name} second call", io=b.io_name)


def test_noalloc_split_counts_and_f32_partials():
    # explicit split counts (more pieces per segment), and the f32 cache whose
    # VALU kernels keep their split partials in the same scratch
    for dtype, splits in (("bf16", 3), ("bf16", 7), ("f32", 4), ("f32", 0)):
        w = DecodeWorkload("noalloc" + dtype, 5, 8, 2, 64, dtype, (1, 700))
        b = Built(w)
        q = torch.from_numpy(w.q()).to(b.io).cuda()
        y = _check_pair(b, b.seqs, q, num_splits=splits)
        assert_close(f64(y), b.oracle_decode(q), what=f"{dtype} splits={splits}", io=b.io_name)
        y2 = _check_pair(b, b.seqs[:2].contiguous(), q[:2].contiguous(), num_splits=splits)
        assert_close(f64(y2), b.oracle_decode(q)[:2], what=f"{dtype} second", io=b.io_name)


def test_noalloc_rejects_plans_beyond_the_scratch():
    # one live sequence; a 1,000-entry batch needs 1,000 x 8 segments of
    # 16 x 130 floats plus the chip's waves: more than 64 MiB.  Rejected on
    # the host, before anything is enqueued; `out` keeps its contents.
    c = kv.KvCache(1, 32, 8, 128, 4, 1, 4, "bf16")
    c.seq_alloc(0, 5)
    n = 1000
    assert c.decode_workspace_bytes(n) > 64 << 20
    seqs = torch.zeros(n, dtype=torch.int32, device="cuda")
    q = torch.zeros((n, 32, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.full((n, 32, 128), 3.0, dtype=torch.bfloat16, device="cuda")
    rc = kv.lib().kvc_attn_decode_noalloc(c._h, 0, n, ctypes.c_void_p(seqs.data_ptr()),
                                          ctypes.c_void_p(q.data_ptr()),
                                          ctypes.c_void_p(out.data_ptr()), ctypes.c_float(0.1),
                                          0, ctypes.c_void_p(0))
    torch.cuda.synchronize()
    assert rc == kv.KVC_E_WORKSPACE
    assert b"64 MiB" in kv.lib().kvc_last_error() or b"library scratch" in kv.lib().kvc_last_error()
    assert bool((out.float() == 3.0).all())
