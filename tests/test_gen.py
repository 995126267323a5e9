"""The seeded generators: same seed -> same bytes, any chunk on its own."""
import numpy as np

import gen


def test_chunk_addressable_and_deterministic():
    for name in ("c1", "c2", "c5"):
        w = gen.get(name)
        a = gen.kv_rows(w, 0, 4000, 8300)
        b = gen.kv_rows(w, 0, 4096, 8200, threads=False)
        assert np.array_equal(a[96:4200], b)
        assert np.array_equal(gen.idx_k_rows(w, 0, 10, 20), gen.idx_k_rows(w, 0, 0, 30)[10:20])
        assert np.array_equal(gen.attn_q(w, 0, 0, 1), gen.attn_q(w, 0)[:1])


def test_dtypes_and_distributions():
    w = gen.get("c2")
    ik = gen.idx_k_rows(w, 3, 0, 4096)
    assert np.array_equal(gen.bf16_round(ik), ik)
    kv = gen.kv_rows(w, 3, 0, 4096)
    big = np.sort(np.argsort(kv.std(0))[-5:])
    assert np.all(kv.std(0)[big] > 10) and np.all(np.delete(kv.std(0), big) < 1.2)
    lens = gen.seq_lens(w)
    assert lens.min() >= 32768 and lens.max() <= 65536 and len(lens) == 32
    c1 = gen.get("c1")
    q = gen.attn_q(c1, 0)
    assert q.shape == (1, 16, 512) and abs(q.std() * np.sqrt(512) - 1) < 0.05


def test_drift_is_a_random_walk():
    w = gen.get("c5").scaled(n=8 * gen.CHUNK)
    x = gen.idx_k_rows(w, 1, 0, w.n).astype(np.float64)
    # increments of the slow mean: windowed means drift with variance ~ sigma^2 * lag
    m = x.reshape(-1, 1024, 64).mean(1)
    d = np.diff(m, axis=0)
    assert 0.5 < d.std() / (0.01 * np.sqrt(1024)) < 1.6


def test_benchmark_accounting_of_the_variants():
    """Algorithmic bytes per step: bf16 keys 128 B, MXFP4 keys 34 B per scanned entry; the
    verification workload scans each sequence's keys once and attends 5 rows per sequence."""
    import bench
    w = gen.get("c3")
    lens = gen.seq_lens(w)
    b = bench.algorithmic_bytes(w, lens)
    m = bench.algorithmic_bytes(w, lens, mxfp4=True)
    assert b["index_scan"] == int(lens.sum()) * 128
    assert m["index_scan"] == int(lens.sum()) * 34
    assert b["reindex_score"] == 2 * 16 * 8192 * 128 and m["reindex_score"] == 2 * 16 * 8192 * 34
    assert b["attention_per_layer"] == 16 * (2048 * 288 + 2048 * 4 + 64 * 512 * 2 + 64 * 512 * 4)
    v = gen.get("c3v")
    bv = bench.algorithmic_bytes(v, gen.seq_lens(v))
    assert v.rows == 80 and bv["index_scan"] == b["index_scan"]
    assert bv["attention_per_layer"] == 5 * b["attention_per_layer"]
    assert bench.index_flops(v, gen.seq_lens(v)) == 5 * bench.index_flops(w, lens)
