"""The benchmark's work accounting (FLOPs per step) against closed forms: the
main-attention work ratio Lk/L^2 = 2048/128000 = 0.016 of the cost discussion
on the DSA technical-report reading (sections "Стоимость" and its exercise),
and the causal pair counts of the prefill configurations."""
import numpy as np

import bench
import synth


def test_main_attention_ratio_at_128k():
    L, k = 128000, 2048
    nvis = np.full(L, L, dtype=np.int64)  # every query sees the whole context
    ratio = bench.mla_flops(nvis, k) / bench.dense_mla_flops(nvis)
    assert abs(ratio - 0.016) < 1e-12


def test_causal_prefill_counts():
    b = synth.Batch.prefill(32768, 32768, 0)
    nvis = bench.visible_counts(b.cu_q, b.cu_kv, b.pos0)
    assert nvis.sum() == 32768 * 32769 // 2
    sel = np.minimum(nvis, 2048).sum()
    assert sel == 2048 * 32768 - 2048 * 2047 // 2
    assert abs(bench.mla_flops(nvis, 2048) - sel * 128 * 2 * (576 + 512)) < 1
    assert abs(bench.indexer_flops(nvis) - 2 * 64 * 128 * nvis.sum()) < 1
    # chunked prefill at the end of 128K: rows see 126977 .. 131072 keys
    c = synth.Batch.prefill(4096, 131072, 126976)
    nv = bench.visible_counts(c.cu_q, c.cu_kv, c.pos0)
    assert nv[0] == 126977 and nv[-1] == 131072


def test_decode_counts():
    b = synth.Batch.decode([16384, 131072, 70000])
    nvis = bench.visible_counts(b.cu_q, b.cu_kv, b.pos0)
    assert nvis.tolist() == [16384, 131072, 70000]
