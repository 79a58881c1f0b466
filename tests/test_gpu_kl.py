"""GPU parity of the indexer KL loss (dsa_indexer_kl_fwd) against the oracle:
page "Техотчёт DeepSeek-V3.2 (2025): разреженное внимание DSA и
масштабирование RL", section "Как учили индексатор" — the target is the main
attention summed over heads and L1-normalised, the loss KL(target || softmax
of the index scores), over every visible key (dense warm-up) or the selected
keys (sparse stage).

Every input of the GPU call comes from the oracle or the input generator: the
index scores (oracle indexer), the selections (oracle top-k, or hand-made with
holes), and the attention's lse (oracle attention over the same set, rounded
to fp32, which is what the kernel takes as input).  The oracle's own loss uses
its exact double-precision softmax.

Tolerance: the loss is a sum of about n = 2048 fp32 terms built from fp32
logits (bf16 products accumulated in fp32: relative error ~1e-6) through
exp2/log2; |kl_gpu - kl_ref| <= 1e-3 * |kl_ref| + 1e-4 (the indexer-score
tolerance of the hot path, with an absolute floor for losses near 0), and the
target p per slot within 1e-3 relative + 1e-9.
"""
import numpy as np
import pytest
import torch

import bench
import oracle
import synth
from gpu_util import dev, say

pytestmark = pytest.mark.gpu

KL_RTOL, KL_ATOL = 1e-3, 1e-4
P_RTOL, P_ATOL = 1e-3, 1e-9


@pytest.fixture(scope="module")
def dsa():
    import sparse_attention_16_amd as m  # fails loudly when libdsa.so is missing
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def _scores(inp, rows=None, ld=None):
    b = inp.batch
    return oracle.indexer(b.cu_q, b.cu_kv, b.pos0, inp.qi, inp.qi_scale, inp.w, inp.ki, inp.ki_scale,
                          rows=rows, ld=ld)


def _check(kl_gpu, kl_ref, p_gpu=None, p_ref=None, what=""):
    err = np.abs(kl_gpu.astype(np.float64) - kl_ref)
    bad = err > KL_RTOL * np.abs(kl_ref) + KL_ATOL
    assert not np.any(bad), f"{what}: {bad.sum()} rows out of tolerance, worst {err.max():.3g}"
    if p_ref is not None:
        m = ~np.isnan(p_ref)
        perr = np.abs(p_gpu[m].astype(np.float64) - p_ref[m])
        pbad = perr > P_RTOL * np.abs(p_ref[m]) + P_ATOL
        assert not np.any(pbad), f"{what}: {pbad.sum()} target values out of tolerance, worst {perr.max():.3g}"
    rel = err / np.maximum(np.abs(kl_ref), 1e-30)
    return float(err.max()) if err.size else 0.0, float(rel.max()) if rel.size else 0.0


def _run(dsa, inp, scores, lse, idx=None, want_p=True):
    b = inp.batch
    batch = dsa.Batch.from_host(b.cu_q, b.cu_kv, b.pos0)
    sc = np.nan_to_num(scores, nan=0.0).astype(np.float32)   # columns past a context are never read
    ld = sc.shape[1]
    kl = torch.empty(b.T, dtype=torch.float32, device="cuda")
    width = idx.shape[1] if idx is not None else ld
    p = torch.full((b.T, width), float("nan"), dtype=torch.float32, device="cuda") if want_p else None
    dsa.indexer_kl_fwd(batch, dev(inp.q), dev(inp.kv), dev(lse.astype(np.float32)), inp.scale, dev(sc), kl,
                       idx=dev(idx) if idx is not None else None, p_out=p)
    torch.cuda.synchronize()
    return kl.cpu().numpy(), (p.cpu().numpy() if p is not None else None)


SPARSE_CASES = {
    "prefill_300_k64": lambda: synth.make_inputs(synth.Batch.prefill(300, 300, 0), seed=161, k=64),
    "prefill_700_k2048": lambda: synth.make_inputs(synth.Batch.prefill(700, 700, 0), seed=162, k=2048),
    "ragged_k100": lambda: synth.make_inputs(synth.Batch.ragged([70, 1, 33, 2], [200, 90, 33, 0], [130, 89, 0, 0]),
                                             seed=163, k=100),
    "decode_k2048": lambda: synth.make_inputs(synth.Batch.decode([1, 40, 2049, 9000, 40000]), seed=164, k=2048,
                                              per_seq=True),
}


@pytest.mark.parametrize("name", sorted(SPARSE_CASES))
def test_indexer_kl_sparse_stage(dsa, name):
    say(f"[indexer_kl sparse] {name}")
    inp = SPARSE_CASES[name]()
    b = inp.batch
    scores = _scores(inp)
    idx = oracle.topk(b.cu_q, b.cu_kv, b.pos0, scores, inp.k)
    _, lse = oracle.sparse_attn(b.cu_q, b.cu_kv, b.pos0, inp.q, inp.kv, idx, inp.Dv, inp.scale)
    kl_ref, p_ref = oracle.indexer_kl(b.cu_q, b.cu_kv, b.pos0, inp.q, inp.kv, inp.scale, scores, idx=idx,
                                      want_p=True)
    kl, p = _run(dsa, inp, scores, lse, idx=idx)
    worst, rel = _check(kl, kl_ref, p, p_ref, name)
    say(f"  max |dkl| {worst:.3g} (max rel {rel:.3g}); kl range {kl_ref.min():.3g} .. {kl_ref.max():.3g}")


def test_indexer_kl_sparse_holes_duplicates_and_empty_rows(dsa):
    inp = synth.make_inputs(synth.Batch.prefill(48, 3000, 2952), seed=165, k=300)
    b = inp.batch
    scores = _scores(inp)
    rng = np.random.default_rng(8)
    idx = np.full((48, 300), -1, np.int32)
    for t in range(48):
        n = [0, 1, 31, 32, 33, 299, 300, 150][t % 8]
        idx[t, :n] = rng.choice(2953 + t, n, replace=n > 2953 + t)
    idx[rng.random(idx.shape) < 0.1] = -1      # holes anywhere
    idx[9, :20] = 17                            # one position listed 20 times
    ref_idx = idx.copy()
    bad = idx.copy()
    bad[11, 5] = 3000 + 11 + 5                  # outside the context: skipped like -1
    ref_idx[11, 5] = -1
    _, lse = oracle.sparse_attn(b.cu_q, b.cu_kv, b.pos0, inp.q, inp.kv, ref_idx, inp.Dv, inp.scale)
    kl_ref, p_ref = oracle.indexer_kl(b.cu_q, b.cu_kv, b.pos0, inp.q, inp.kv, inp.scale, scores, idx=ref_idx,
                                      want_p=True)
    kl, p = _run(dsa, inp, scores, lse, idx=bad)
    _check(kl, kl_ref, p, p_ref, "holes")
    assert np.all(kl[0::8] == 0.0) and np.all(p[0::8] == 0.0)   # rows with no slot


DENSE_CASES = {
    "prefill_300": lambda: synth.make_inputs(synth.Batch.prefill(300, 300, 0), seed=171, k=2048),
    "chunked_40_at_960": lambda: synth.make_inputs(synth.Batch.prefill(40, 1000, 960), seed=172, k=2048),
    "ragged_empty_cache": lambda: synth.make_inputs(
        synth.Batch.ragged([70, 1, 33, 3], [200, 90, 33, 0], [130, 89, 0, 0]), seed=173, k=2048),
    # few rows over long contexts: the slot range is split over workgroups
    "decode_long": lambda: synth.make_inputs(synth.Batch.decode([1, 17, 3000, 12000]), seed=174, k=2048,
                                             per_seq=True),
}


@pytest.mark.parametrize("name", sorted(DENSE_CASES))
def test_indexer_kl_dense_stage(dsa, name):
    say(f"[indexer_kl dense] {name}")
    inp = DENSE_CASES[name]()
    b = inp.batch
    scores = _scores(inp)
    _, lse = oracle.dense_attn(b.cu_q, b.cu_kv, b.pos0, inp.q, inp.kv, inp.Dv, inp.scale)
    kl_ref, p_ref = oracle.indexer_kl(b.cu_q, b.cu_kv, b.pos0, inp.q, inp.kv, inp.scale, scores, want_p=True)
    kl, p = _run(dsa, inp, scores, lse)
    worst, rel = _check(kl, kl_ref, p, p_ref, name)
    say(f"  max |dkl| {worst:.3g} (max rel {rel:.3g}); kl range {kl_ref.min():.3g} .. {kl_ref.max():.3g}")


def test_indexer_kl_without_target_output(dsa):
    # the direct path (one workgroup per row, no target written) gives the same loss
    inp = synth.make_inputs(synth.Batch.prefill(600, 600, 0), seed=175, k=256)
    b = inp.batch
    scores = _scores(inp)
    idx = oracle.topk(b.cu_q, b.cu_kv, b.pos0, scores, inp.k)
    _, lse = oracle.sparse_attn(b.cu_q, b.cu_kv, b.pos0, inp.q, inp.kv, idx, inp.Dv, inp.scale)
    kl_ref = oracle.indexer_kl(b.cu_q, b.cu_kv, b.pos0, inp.q, inp.kv, inp.scale, scores, idx=idx)
    kl, _ = _run(dsa, inp, scores, lse, idx=idx, want_p=False)
    _check(kl, kl_ref, what="no target")


def test_indexer_kl_32k_sparse_stage_sampled(dsa):
    """The 32K-prefill sparse stage bench.py times (indexer_kl_32k): every
    row runs; sampled rows carry oracle inputs and are checked."""
    say("[fullsize] indexer_kl_32k")
    wl, _ = bench.make_workload("prefill_32k")
    b = wl.batch
    d = wl.device("cuda")
    rows = np.array([0, 1, 2046, 2047, 2048, 2049, 16000, 32767])
    inp = wl.sampled_host(rows)
    ld = ((b.max_kv + 63) // 64) * 64
    s_rows = oracle.indexer(b.cu_q, b.cu_kv, b.pos0, inp.qi, inp.qi_scale, inp.w, inp.ki, inp.ki_scale, rows=rows,
                            ld=ld)
    idx_rows = oracle.topk(b.cu_q, b.cu_kv, b.pos0, s_rows, wl.k, rows=rows)
    _, lse_rows = oracle.sparse_attn(b.cu_q, b.cu_kv, b.pos0, inp.q, inp.kv, idx_rows, wl.Dv, wl.scale, rows=rows)
    kl_ref = oracle.indexer_kl(b.cu_q, b.cu_kv, b.pos0, inp.q, inp.kv, wl.scale, s_rows, idx=idx_rows, rows=rows)
    # full-size inputs: the sampled rows from the oracle, the others a valid filler
    scores = torch.zeros((b.T, ld), dtype=torch.float32, device="cuda")
    idx = torch.full((b.T, wl.k), -1, dtype=torch.int32, device="cuda")
    idx[:, 0] = 0
    lse = torch.zeros((b.T, 128), dtype=torch.float32, device="cuda")
    r = torch.as_tensor(rows, device="cuda")
    scores[r] = dev(np.nan_to_num(s_rows, nan=0.0).astype(np.float32))
    idx[r] = dev(idx_rows)
    lse[r] = dev(lse_rows)
    batch = dsa.Batch.from_host(b.cu_q, b.cu_kv, b.pos0)
    kl = torch.empty(b.T, dtype=torch.float32, device="cuda")
    dsa.indexer_kl_fwd(batch, d["q"], d["kv"], lse, wl.scale, scores, kl, idx=idx)
    torch.cuda.synchronize()
    worst, rel = _check(kl[r].cpu().numpy(), kl_ref, what="32k sampled")
    say(f"  32k: max |dkl| {worst:.3g} (max rel {rel:.3g})")
