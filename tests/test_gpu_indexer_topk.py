"""GPU parity of the fused indexer + select (dsa_indexer_topk, the first half of
the fused entries): the top-k positions straight from the indexer inputs, with
no score matrix in memory (page "Техотчёт DeepSeek-V3.2 (2025): разреженное
внимание DSA и масштабирование RL", sections "Молниеносный индексатор" and
"Отбор и основное внимание").

Two references:
  * dsa_indexer_scores + dsa_topk on the same inputs: the scores are the same
    fp32 values (same arithmetic), so the selection must be identical bit for
    bit, on every row;
  * the oracle's top-k of its own scores: identical sets except near-ties of the
    k-th score (the tolerances of tests/gpu_util.py).
The recompute path (rows whose sampled threshold cannot prove the candidate
set complete) is forced two ways: every key of a row with the same score (more
candidates than one select holds), and keys that score above zero only on the
positions the threshold samples (the threshold lands above the k-th score).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import DevInputs, check_idx_sets, dev, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsa():
    import sparse_attention_16_amd as m  # fails loudly when libdsa.so is missing
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def _three_steps(dsa, d, b, k):
    ld = ((b.max_kv + 63) // 64) * 64
    scores = torch.empty((b.T, ld), device="cuda")
    dsa.indexer_scores(d.batch, d.qi, d.qs, d.w, d.ki, d.ks, scores)
    idx3 = torch.full((b.T, k), -9, dtype=torch.int32, device="cuda")
    dsa.topk(d.batch, scores, k, idx3)
    return idx3


CASES = {
    # every row sees at most 4096 keys: no threshold, every visible key is a candidate
    "prefill_600_k128": lambda: synth.make_inputs(synth.Batch.prefill(600, 600, 0), seed=151, k=128),
    # sampled thresholds, one candidate region per row (whole-row indexer workgroups)
    "prefill_40_at_9000_k2048": lambda: synth.make_inputs(synth.Batch.prefill(40, 9040, 9000), seed=152, k=2048),
    "ragged_k64": lambda: synth.make_inputs(
        synth.Batch.ragged([70, 1, 33, 5], [6000, 90, 33, 20000], [5900, 89, 0, 19990]), seed=153, k=64),
    # decode layout: 512-column regions, rows of 1 .. 131072 keys
    "decode_mixed_k2048": lambda: synth.make_inputs(
        synth.Batch.decode([1, 2048, 2049, 4097, 9000, 32768, 32769, 70001, 131072]), seed=154, k=2048,
        per_seq=True),
    "decode_small_k7": lambda: synth.make_inputs(synth.Batch.decode([5, 7, 8, 5000, 40000]), seed=155, k=7,
                                                 per_seq=True),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_indexer_topk_matches_three_steps_and_oracle(dsa, name):
    say(f"[indexer_topk] {name}")
    inp = CASES[name]()
    b = inp.batch
    d = DevInputs(inp, dsa)
    idx = torch.full((b.T, inp.k), -7, dtype=torch.int32, device="cuda")
    dsa.indexer_topk(d.batch, d.qi, d.qs, d.w, d.ki, d.ks, inp.k, idx)
    idx3 = _three_steps(dsa, d, b, inp.k)
    torch.cuda.synchronize()
    g, g3 = idx.cpu().numpy(), idx3.cpu().numpy()
    assert np.array_equal(g, g3), f"{name}: {np.sum(np.any(g != g3, axis=1))} rows differ from the three steps"
    rows = np.arange(b.T) if b.T <= 64 else np.unique(np.linspace(0, b.T - 1, 64).astype(np.int64))
    ref_s, A = oracle.indexer(b.cu_q, b.cu_kv, b.pos0, inp.qi, inp.qi_scale, inp.w, inp.ki, inp.ki_scale,
                              rows=rows, want_abs=True)
    ref_idx = oracle.topk(b.cu_q, b.cu_kv, b.pos0, ref_s, inp.k, rows=rows)
    _, _, _, _, nvis = oracle.visible(b.cu_q, b.cu_kv, b.pos0)
    differ = check_idx_sets(g[rows], ref_idx, ref_s, A, nvis[rows], inp.k, name)
    say(f"  {b.T} rows identical to the three steps; {len(rows)} checked against the oracle, "
        f"{len(differ)} differ only at near-ties")


def _sample_grid(n, seq):
    """Positions the threshold samples for a one-row sequence of n visible keys
    (the sample kernel's grid: m = clamp(n // 32, 512, 1024) keys at stride
    n // m from an offset hashed from the row block (0) and the sequence)."""
    m = min(max(n // 32, 512), 1024)
    stride = n // m
    o = ((0 * 2654435761 + seq * 40503) & 0xFFFFFFFF) % stride
    return o + stride * np.arange(m)


def test_indexer_topk_recompute_threshold_too_high(dsa):
    """Keys score above zero only on the sampled positions (non-negative head
    weights, zero key rows elsewhere): the threshold, a high rank of the
    sample, exceeds the k-th largest score (most of the top k are zeros), so
    fewer than k keys reach it and the rows are recomputed on chip.  The exact
    selection keeps every sampled key and the lowest-positioned zero-score keys
    (exact ties).  Rows of one and of several 32768-column chunks."""
    say("[indexer_topk] recompute: threshold above the k-th score")
    ctx = [9000, 32768, 50000, 131072]
    inp = synth.make_inputs(synth.Batch.decode(ctx), seed=156, k=2048, per_seq=True)
    b = inp.batch
    inp.w[:] = np.abs(inp.w)
    keep = np.zeros(b.N, bool)
    for sq, n in enumerate(ctx):
        keep[int(b.cu_kv[sq]) + _sample_grid(n, sq)] = True
    inp.ki[~keep] = 0
    inp.ki_scale[~keep] = 1.0
    d = DevInputs(inp, dsa)
    idx = torch.full((b.T, inp.k), -7, dtype=torch.int32, device="cuda")
    dsa.indexer_topk(d.batch, d.qi, d.qs, d.w, d.ki, d.ks, inp.k, idx)
    idx3 = _three_steps(dsa, d, b, inp.k)
    torch.cuda.synchronize()
    g, g3 = idx.cpu().numpy(), idx3.cpu().numpy()
    ref_s = oracle.indexer(b.cu_q, b.cu_kv, b.pos0, inp.qi, inp.qi_scale, inp.w, inp.ki, inp.ki_scale)
    ref = oracle.topk(b.cu_q, b.cu_kv, b.pos0, ref_s, inp.k)
    for sq, n in enumerate(ctx):
        pos = np.sort(_sample_grid(n, sq))
        assert np.all(ref_s[sq, pos] > 0) and np.all(np.delete(ref_s[sq, :n], pos) == 0)
        assert np.all(np.isin(pos, ref[sq]))    # the case is what it claims: every sampled key selected
    assert np.array_equal(g3, ref), "three steps against the oracle"
    assert np.array_equal(g, ref), f"{np.sum(np.any(g != ref, axis=1))} rows differ from the oracle"
    say(f"  {b.T} rows recomputed, identical to the oracle and the three steps")


def test_indexer_topk_recompute_all_equal_scores(dsa):
    """Every key row the same: each row's scores are all equal, every visible
    key reaches the threshold, and rows longer than one select's register
    capacity (16384 candidates) are recomputed; the exact ties select the k
    lowest positions.  Prefill-shaped and decode-shaped batches."""
    say("[indexer_topk] recompute: all scores equal")
    # (up to 1024 rows: the workgroup select queues a row for the recompute
    # kernel; 1100 rows: the wave select hands it to the workgroup select,
    # which queues it)
    for name, bt in (("decode", synth.Batch.decode([3000, 16384, 16385, 40000])),
                     ("prefill", synth.Batch.prefill(20, 20000, 19980)),
                     ("prefill_300", synth.Batch.prefill(300, 20000, 19700)),
                     ("prefill_1100", synth.Batch.prefill(1100, 18000, 16900))):
        inp = synth.make_inputs(bt, seed=157, k=2048, per_seq=(name == "decode"))
        b = inp.batch
        inp.ki[:] = inp.ki[0]
        inp.ki_scale[:] = inp.ki_scale[0]
        d = DevInputs(inp, dsa)
        idx = torch.full((b.T, inp.k), -7, dtype=torch.int32, device="cuda")
        dsa.indexer_topk(d.batch, d.qi, d.qs, d.w, d.ki, d.ks, inp.k, idx)
        torch.cuda.synchronize()
        g = idx.cpu().numpy()
        _, _, _, _, nvis = oracle.visible(b.cu_q, b.cu_kv, b.pos0)
        for r in range(b.T):
            m = min(int(nvis[r]), inp.k)
            want = np.concatenate([np.arange(m), np.full(inp.k - m, -1)])
            assert np.array_equal(g[r], want), f"{name} row {r}"
        say(f"  {name}: {b.T} rows select their k lowest positions")


def test_indexer_topk_workspace_and_validation(dsa):
    inp = CASES["prefill_600_k128"]()
    d = DevInputs(inp, dsa)
    need = dsa.workspace_size(dsa.WS_INDEXER_TOPK, d.batch, inp.k)
    assert need > 0
    idx = torch.empty((inp.batch.T, inp.k), dtype=torch.int32, device="cuda")
    small = torch.empty(need - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(dsa.DsaError) as e:
        dsa.indexer_topk(d.batch, d.qi, d.qs, d.w, d.ki, d.ks, inp.k, idx, ws=small)
    assert e.value.status == dsa.DSA_ERR_WORKSPACE


def _wave_case(name):
    """Batches of more than 4 rows per compute unit, which take the select with
    one wave per row: 1100 query rows at the end of a context."""
    if name == "spread":          # ~3k candidates per row: the histogram path
        return synth.make_inputs(synth.Batch.prefill(1100, 6000, 4900), seed=161, k=2048), None
    if name == "ties_1000":       # every score repeated ~6 times: exact ties around the k-th
        return synth.make_inputs(synth.Batch.prefill(1100, 6000, 4900), seed=162, k=2048), 1000
    if name == "ties_3_k64":      # three distinct scores per row: candidates all equal, no value bins
        return synth.make_inputs(synth.Batch.prefill(1100, 6000, 4900), seed=163, k=64), 3
    if name == "long_rows":       # ~4k+ candidates per row: more than one wave holds, the workgroup select
        return synth.make_inputs(synth.Batch.prefill(1100, 90000, 88900), seed=164, k=2048), None
    raise KeyError(name)


@pytest.mark.parametrize("name", ["spread", "ties_1000", "ties_3_k64", "long_rows"])
def test_indexer_topk_wave_select(dsa, name):
    say(f"[indexer_topk wave select] {name}")
    inp, period = _wave_case(name)
    if period is not None:
        inp.ki[:] = inp.ki[np.arange(inp.ki.shape[0]) % period]
        inp.ki_scale[:] = inp.ki_scale[np.arange(inp.ki.shape[0]) % period]
    b = inp.batch
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    assert b.T > 4 * ncu or ncu != 256
    d = DevInputs(inp, dsa)
    idx = torch.full((b.T, inp.k), -7, dtype=torch.int32, device="cuda")
    dsa.indexer_topk(d.batch, d.qi, d.qs, d.w, d.ki, d.ks, inp.k, idx)
    idx3 = _three_steps(dsa, d, b, inp.k)
    torch.cuda.synchronize()
    g, g3 = idx.cpu().numpy(), idx3.cpu().numpy()
    assert np.array_equal(g, g3), f"{name}: {np.sum(np.any(g != g3, axis=1))} rows differ from the three steps"
    rows = np.array([0, 1, 517, b.T - 2, b.T - 1])
    ref_s, A = oracle.indexer(b.cu_q, b.cu_kv, b.pos0, inp.qi, inp.qi_scale, inp.w, inp.ki, inp.ki_scale,
                              rows=rows, want_abs=True)
    ref_idx = oracle.topk(b.cu_q, b.cu_kv, b.pos0, ref_s, inp.k, rows=rows)
    _, _, _, _, nvis = oracle.visible(b.cu_q, b.cu_kv, b.pos0)
    differ = check_idx_sets(g[rows], ref_idx, ref_s, A, nvis[rows], inp.k, name)
    say(f"  {b.T} rows identical to the three steps; {len(differ)} of {len(rows)} oracle rows differ at near-ties")


def test_threshold_keeps_candidates_near_k_without_recompute(dsa):
    """The sampled threshold (the rank-th largest sampled score, rank = mu +
    5 sqrt(mu) + 1) on N(0,1) inputs: no row is recomputed (the threshold is
    never above the k-th score) and the candidates per row stay near the
    expected (rank / mu) k, about 1.6 k here.  A threshold drawn wrong either
    way fails one of the two: too high sends rows to the recompute, too low
    floods the select.  Prefill (wave select) and decode (workgroup select)."""
    say("[threshold] candidates per row and recomputed rows")
    pre = synth.make_inputs(synth.Batch.prefill(1536, 20000, 18464), seed=158, k=2048)
    dec = synth.make_inputs(synth.Batch.decode(synth.decode_contexts(159, 32, 20000, 100000)), seed=159, k=2048,
                            per_seq=True)
    for name, inp, decode in (("prefill", pre, False), ("decode", dec, True)):
        b = inp.batch
        d = DevInputs(inp, dsa)
        args = dsa.fwd_args(d.batch, d.qi, d.qs, d.w, d.ki, d.ks, d.q, d.kv, inp.k, inp.scale)
        out = torch.empty((b.T, inp.H, inp.Dv), dtype=torch.int16, device="cuda")
        lse = torch.empty((b.T, inp.H), device="cuda")
        prof = dsa.fwd_profile(args, d.batch, out, lse, decode=decode)
        items = {name_: it for name_, _, it in prof}
        assert items.get("idx_fallback_kernel") == 0, f"{name}: rows recomputed: {prof}"
        if not decode:
            cands = [it for n_, _, it in prof if n_.startswith("cand_select_wave")]
            assert cands, prof
            per_row = cands[0] / b.T
            say(f"  {name}: {per_row:.0f} candidates per row, none recomputed")
            assert 1.2 * inp.k <= per_row <= 2.2 * inp.k, per_row
        else:
            say(f"  {name}: none recomputed")
