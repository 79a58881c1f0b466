"""GPU parity of the short-sequence mode, the "MHA with mask" of page
"Техотчёт DeepSeek-V3.2 (2025): разреженное внимание DSA и масштабирование RL",
section "Стоимость": for short sequences a masked dense mode stands in for DSA
and gives its result.

* dsa_dense_mla_fwd against the oracle's brute-force causal attention over
  every visible key (small cases: all rows; a 2048-token prompt: sampled rows).
* The fused entries on sequences whose contexts all fit in k switch to this
  mode; their idx, out and lse must be identical, bit for bit, to the three
  separate steps (indexer -> top-k -> sparse attention over the -1 padded
  selection) on the same inputs, and idx must be every visible key in order.
* Rows past the last usable slot of a selection stop early; the sparse path on
  a -1 padded selection is checked against the oracle on the same idx.
"""
import numpy as np
import pytest
import torch

import bench
import oracle
import synth
from gpu_util import DevInputs, bf16_to_f32, check_attention, dev, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsa():
    import sparse_attention_16_amd as m  # fails loudly when libdsa.so is missing
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


DENSE_CASES = {
    # one prompt from position 0 (several 32-key blocks, ragged last block)
    "prefill_300": lambda: synth.make_inputs(synth.Batch.prefill(300, 300, 0), seed=131, k=2048),
    # a chunk at the end of a 1000-row cache: rows see 961..1000 keys
    "chunked_40_at_960": lambda: synth.make_inputs(synth.Batch.prefill(40, 1000, 960), seed=132, k=2048),
    # ragged sequences, one with an empty cache (its rows see nothing)
    "ragged_4seq": lambda: synth.make_inputs(
        synth.Batch.ragged([70, 1, 33, 3], [200, 90, 33, 0], [130, 89, 0, 0]), seed=133, k=2048),
    # few rows: split-KV partials and their merge; contexts 1 and exactly 2048
    "decode_edges": lambda: synth.make_inputs(synth.Batch.decode([1, 17, 300, 2047, 2048]), seed=134,
                                              k=2048, per_seq=True),
}


@pytest.mark.parametrize("name", sorted(DENSE_CASES))
def test_dense_mla_matches_oracle(dsa, name):
    say(f"[dense_mla] {name}")
    inp = DENSE_CASES[name]()
    b = inp.batch
    o_ref, lse_ref = oracle.dense_attn(b.cu_q, b.cu_kv, b.pos0, inp.q, inp.kv, inp.Dv, inp.scale)
    d = DevInputs(inp, dsa)
    out = torch.empty((b.T, inp.H, inp.Dv), dtype=torch.int16, device="cuda")
    lse = torch.empty((b.T, inp.H), dtype=torch.float32, device="cuda")
    dsa.dense_mla_fwd(d.batch, d.q, d.kv, inp.scale, out, lse)
    torch.cuda.synchronize()
    dl, rel = check_attention(bf16_to_f32(out), lse.cpu().numpy(), o_ref, lse_ref, name)
    say(f"  max |dlse| {dl:.3g}, max row ||do||/||o|| {rel:.3g}")


def _three_step(dsa, d, inp):
    b = inp.batch
    ld = ((b.max_kv + 63) // 64) * 64
    scores = torch.empty((b.T, max(ld, 64)), dtype=torch.float32, device="cuda")
    idx = torch.empty((b.T, inp.k), dtype=torch.int32, device="cuda")
    out = torch.empty((b.T, inp.H, inp.Dv), dtype=torch.int16, device="cuda")
    lse = torch.empty((b.T, inp.H), dtype=torch.float32, device="cuda")
    dsa.indexer_scores(d.batch, d.qi, d.qs, d.w, d.ki, d.ks, scores)
    dsa.topk(d.batch, scores, inp.k, idx)
    dsa.sparse_mla_fwd(d.batch, d.q, d.kv, idx, inp.scale, out, lse)
    return idx, out, lse


SHORT_CASES = {
    "prefill_1000_k2048": (lambda: synth.make_inputs(synth.Batch.prefill(1000, 1000, 0), seed=141, k=2048),
                           "prefill"),
    # contexts exactly k: the largest case the mode takes
    "prefill_256_k256": (lambda: synth.make_inputs(synth.Batch.prefill(256, 256, 0), seed=142, k=256),
                         "prefill"),
    "ragged_k100": (lambda: synth.make_inputs(synth.Batch.ragged([50, 7, 30], [100, 7, 64], [50, 0, 34]),
                                              seed=143, k=100), "prefill"),
    "decode_k2048": (lambda: synth.make_inputs(synth.Batch.decode([1, 5, 700, 2048]), seed=144, k=2048,
                                               per_seq=True), "decode"),
}


@pytest.mark.parametrize("name", sorted(SHORT_CASES))
def test_fused_short_mode_equals_three_steps(dsa, name):
    say(f"[short mode] {name}")
    make, entry = SHORT_CASES[name]
    inp = make()
    b = inp.batch
    assert b.max_kv <= inp.k
    d = DevInputs(inp, dsa)
    args = dsa.fwd_args(d.batch, d.qi, d.qs, d.w, d.ki, d.ks, d.q, d.kv, inp.k, inp.scale)
    out = torch.empty((b.T, inp.H, inp.Dv), dtype=torch.int16, device="cuda")
    lse = torch.empty((b.T, inp.H), dtype=torch.float32, device="cuda")
    idx = torch.full((b.T, inp.k), 12345, dtype=torch.int32, device="cuda")
    fn = dsa.prefill_fwd if entry == "prefill" else dsa.decode_fwd
    fn(args, d.batch, out, lse, idx)
    idx3, out3, lse3 = _three_step(dsa, d, inp)
    torch.cuda.synchronize()
    g_idx = idx.cpu().numpy()
    _, _, _, _, nvis = oracle.visible(b.cu_q, b.cu_kv, b.pos0)
    cols = np.arange(inp.k)[None, :]
    want = np.where(cols < nvis[:, None], cols, -1).astype(np.int32)
    assert np.array_equal(g_idx, want), "short-mode idx is not every visible key in order"
    assert np.array_equal(idx3.cpu().numpy(), want), "top-k of a short row is not every visible key"
    assert torch.equal(out, out3), "out differs from the three-step path"
    assert torch.equal(lse.view(torch.int32), lse3.view(torch.int32)), "lse differs from the three-step path"
    # and against the oracle's DSA (scores -> top-k -> exact attention)
    o_ref, lse_ref = oracle.dense_attn(b.cu_q, b.cu_kv, b.pos0, inp.q, inp.kv, inp.Dv, inp.scale)
    dl, rel = check_attention(bf16_to_f32(out), lse.cpu().numpy(), o_ref, lse_ref, name)
    say(f"  identical to the three steps; max |dlse| {dl:.3g}, max row ||do||/||o|| {rel:.3g}")


def test_sparse_mla_padded_selection_stops_early(dsa):
    """Selections with -1 padding after n < k entries (and a row of only
    padding) give the oracle's result on the same idx."""
    inp = synth.make_inputs(synth.Batch.prefill(64, 3000, 2936), seed=151, k=2048)
    b = inp.batch
    rng = np.random.default_rng(3)
    idx = np.full((64, 2048), -1, np.int32)
    for t in range(64):
        n = [1, 31, 32, 33, 700, 2047, 2048, 0][t % 8]
        if n:
            idx[t, :n] = np.sort(rng.choice(2937 + t, n, replace=False))
    o_ref, lse_ref = oracle.sparse_attn(b.cu_q, b.cu_kv, b.pos0, inp.q, inp.kv, idx, inp.Dv, inp.scale)
    d = DevInputs(inp, dsa)
    out = torch.empty((64, 128, 512), dtype=torch.int16, device="cuda")
    lse = torch.empty((64, 128), device="cuda")
    dsa.sparse_mla_fwd(d.batch, d.q, d.kv, dev(idx), inp.scale, out, lse)
    torch.cuda.synchronize()
    dl, rel = check_attention(bf16_to_f32(out), lse.cpu().numpy(), o_ref, lse_ref, "padded")
    assert np.all(np.isneginf(lse.cpu().numpy()[7::8]))
    say(f"  padded selections: max |dlse| {dl:.3g}, max row ||do||/||o|| {rel:.3g}")


def test_short_prefill_2k_fullsize_sampled(dsa):
    """The 2048-token prompt bench.py times (short_prefill_2k) through
    dsa_prefill_fwd, sampled rows against the oracle's dense attention."""
    say("[fullsize] short_prefill_2k")
    wl, entry = bench.make_workload("short_prefill_2k")
    b = wl.batch
    d = wl.device("cuda")
    batch = dsa.Batch.from_host(b.cu_q, b.cu_kv, b.pos0)
    args = dsa.fwd_args(batch, d["qi"], d["qs"], d["w"], d["ki"], d["ks"], d["q"], d["kv"], wl.k, wl.scale)
    out = torch.empty((b.T, 128, 512), dtype=torch.int16, device="cuda")
    lse = torch.empty((b.T, 128), device="cuda")
    idx = torch.empty((b.T, wl.k), dtype=torch.int32, device="cuda")
    dsa.prefill_fwd(args, batch, out, lse, idx)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 31, 32, 33, 1000, 2046, 2047])
    inp = wl.sampled_host(rows)
    o_ref, lse_ref = oracle.dense_attn(b.cu_q, b.cu_kv, b.pos0, inp.q, inp.kv, wl.Dv, wl.scale, rows=rows)
    rsel = torch.as_tensor(rows, device="cuda")
    dl, rel = check_attention(bf16_to_f32(out[rsel]), lse[rsel].cpu().numpy(), o_ref, lse_ref, "short 2k")
    g_idx = idx[rsel].cpu().numpy()
    for r, t in enumerate(rows):
        assert np.array_equal(g_idx[r, :t + 1], np.arange(t + 1)) and np.all(g_idx[r, t + 1:] == -1)
    say(f"  short 2k: max |dlse| {dl:.3g}, max row ||do||/||o|| {rel:.3g}")
