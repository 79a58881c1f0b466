"""The library's debug mode on the GPU.

* DSA_DEBUG_CHECKS=1 validates every selection an entry produces (dsa_topk,
  dsa_indexer_topk, the fused prefill and decode entries, the short mode)
  on the device: on correct outputs each call returns DSA_OK and, with
  DSA_LOG=1, logs how many rows it checked.
* dsa_check_selection itself: 0 on a correct selection, and each row
  corrupted in one of the ways the contract forbids (out of order, out of
  range, a hole before the end, a position where -1 belongs, a repeat) is
  counted once.  The corruptions are made on the host copy of a correct
  selection; the kernel only reads idx.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import DevInputs, dev, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsa():
    import sparse_attention_16_amd as m  # fails loudly when libdsa.so is missing
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def _ragged():
    # rows that see more than k keys (with and without a sampled threshold)
    # and rows that see fewer
    return synth.make_inputs(synth.Batch.ragged([40, 30, 20], [9000, 3000, 600], [8960, 2970, 580]), seed=191,
                             k=2048)


def test_debug_checks_on_every_selecting_entry(dsa, capfd, monkeypatch):
    say("[debug checks] prefill, decode, topk, indexer_topk, short mode")
    monkeypatch.setenv("DSA_DEBUG_CHECKS", "1")
    monkeypatch.setenv("DSA_LOG", "1")
    inp = _ragged()
    b = inp.batch
    d = DevInputs(inp, dsa)
    args = dsa.fwd_args(d.batch, d.qi, d.qs, d.w, d.ki, d.ks, d.q, d.kv, inp.k, inp.scale)
    out = torch.empty((b.T, inp.H, inp.Dv), dtype=torch.int16, device="cuda")
    lse = torch.empty((b.T, inp.H), device="cuda")
    idx = torch.empty((b.T, inp.k), dtype=torch.int32, device="cuda")
    dsa.prefill_fwd(args, d.batch, out, lse, idx)
    dsa.indexer_topk(d.batch, d.qi, d.qs, d.w, d.ki, d.ks, inp.k, idx)
    ld = ((b.max_kv + 63) // 64) * 64
    scores = torch.empty((b.T, ld), device="cuda")
    dsa.indexer_scores(d.batch, d.qi, d.qs, d.w, d.ki, d.ks, scores)
    dsa.topk(d.batch, scores, inp.k, idx)
    torch.cuda.synchronize()
    err = capfd.readouterr().err
    for entry in ("indexer_topk", "dsa_indexer_topk", "dsa_topk"):
        assert f"[dsa] {entry}: debug check: {b.T} rows ok" in err, err
    assert "prefill plan: candidate regions" in err, err

    dec = synth.make_inputs(synth.Batch.decode([1, 2048, 5000, 40000]), seed=192, k=2048, per_seq=True)
    dd = DevInputs(dec, dsa)
    dargs = dsa.fwd_args(dd.batch, dd.qi, dd.qs, dd.w, dd.ki, dd.ks, dd.q, dd.kv, dec.k, dec.scale)
    dout = torch.empty((4, dec.H, dec.Dv), dtype=torch.int16, device="cuda")
    dlse = torch.empty((4, dec.H), device="cuda")
    didx = torch.empty((4, dec.k), dtype=torch.int32, device="cuda")
    dsa.decode_fwd(dargs, dd.batch, dout, dlse, didx)

    short = synth.make_inputs(synth.Batch.prefill(300, 300, 0), seed=193, k=512)
    sd = DevInputs(short, dsa)
    sargs = dsa.fwd_args(sd.batch, sd.qi, sd.qs, sd.w, sd.ki, sd.ks, sd.q, sd.kv, short.k, short.scale)
    sout = torch.empty((300, short.H, short.Dv), dtype=torch.int16, device="cuda")
    slse = torch.empty((300, short.H), device="cuda")
    sidx = torch.empty((300, short.k), dtype=torch.int32, device="cuda")
    dsa.prefill_fwd(sargs, sd.batch, sout, slse, sidx)
    torch.cuda.synchronize()
    err = capfd.readouterr().err
    assert "decode plan: candidate regions" in err and "[dsa] indexer_topk: debug check: 4 rows ok" in err, err
    assert "short mode" in err and "[dsa] select_all_visible: debug check: 300 rows ok" in err, err
    say("  every selecting entry passed its debug check")


def test_check_selection_counts_broken_rows(dsa):
    say("[check_selection] correct selection, then five kinds of corrupted rows")
    inp = _ragged()
    b = inp.batch
    d = DevInputs(inp, dsa)
    k = inp.k
    idx = torch.empty((b.T, k), dtype=torch.int32, device="cuda")
    dsa.indexer_topk(d.batch, d.qi, d.qs, d.w, d.ki, d.ks, k, idx)
    torch.cuda.synchronize()
    assert dsa.check_selection(d.batch, idx) == 0
    _, _, _, _, nvis = oracle.visible(b.cu_q, b.cu_kv, b.pos0)
    full = [r for r in range(b.T) if nvis[r] > k]
    part = [r for r in range(b.T) if 2 < nvis[r] < k]
    assert len(full) >= 3 and len(part) >= 2
    h = idx.cpu().numpy()
    bad_rows = []
    r = full[0]; h[r, [10, 11]] = h[r, [11, 10]]; bad_rows.append(r)          # out of order
    r = full[1]; h[r, k - 1] = nvis[r]; bad_rows.append(r)                    # past the visible keys
    r = full[2]; h[r, 5] = h[r, 4]; bad_rows.append(r)                        # a repeat
    r = part[0]; h[r, 1] = -1; bad_rows.append(r)                             # a hole before the end
    r = part[1]; h[r, nvis[r]] = 0; bad_rows.append(r)                        # a position where -1 belongs
    assert dsa.check_selection(d.batch, dev(h)) == len(bad_rows)
    say(f"  {len(bad_rows)} corrupted rows of {b.T} counted")
