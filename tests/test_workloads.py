"""The seeded generators: shapes, determinism, chunk independence."""
import numpy as np

from workloads import GPT2Small, decode_workload, prefill_workload


def test_decode_workloads_shapes_and_determinism():
    for name in ("llama8b_decode", "llama70b_decode_bf16", "llama70b_decode_fp8",
                 "long_mha_decode"):
        w = decode_workload(name, small=True)
        assert w.q().shape == (w.batch, w.n_q, w.d)
        k, v = w.kv_rows(0, 0, int(w.lengths[0]))
        assert k.shape == (w.lengths[0], w.n_kv, w.d) and k.dtype == np.float32
        k2, _ = decode_workload(name, small=True).kv_rows(0, 0, int(w.lengths[0]))
        assert np.array_equal(k, k2)
        tabs = w.block_tables()
        allb = np.concatenate(tabs)
        assert sorted(allb.tolist()) == list(range(w.n_blocks))
        assert [len(t) for t in tabs] == list(w.blocks_per_seq)


def test_chunked_rows_are_position_addressed():
    w = decode_workload("long_mha_decode", small=True)
    k, v = w.kv_rows(0, 0, 2085)
    k2, v2 = w.kv_rows(0, 1000, 100)
    assert np.array_equal(k[1000:1100], k2) and np.array_equal(v[1000:1100], v2)


def test_full_size_recipes():
    w = decode_workload("llama8b_decode")
    assert w.batch == 40 and w.lengths.min() >= 512 and w.lengths.max() <= 4096
    w = decode_workload("llama70b_decode_fp8")
    assert (w.batch, w.n_q, w.n_kv, int(w.lengths[0])) == (8, 64, 8, 32768)
    k, _ = w.kv_rows(0, 0, 4096)
    frac = np.mean(np.abs(k) > 6)          # outliers (x8) dominate |x| > 6
    assert 0.004 < frac < 0.02
    w = decode_workload("long_mha_decode")
    assert (w.n_q, w.n_kv, int(w.lengths[0])) == (32, 32, 128000)
    p = prefill_workload()
    assert (p.batch, p.T, p.n_q, p.n_kv, p.d) == (4, 8192, 32, 8, 128)


def test_gpt2_small_recipe():
    w = GPT2Small(n_new=3)
    assert w.q_prompt.shape == (261, 12, 64) and len(w.steps) == 3
    assert abs(np.std(w.k_prompt) - 1.0) < 0.1      # x W with W ~ N(0,1)/sqrt(768)
