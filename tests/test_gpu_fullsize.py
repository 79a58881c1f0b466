"""GPU parity at the full DSA configuration sizes, in the launch configuration
bench.py times (dsa_prefill_fwd for prefill workloads, dsa_decode_fwd for the
decode batch), checked on sampled query rows that the oracle recomputes one by
one: index scores (through dsa_indexer_scores on the same inputs), the top-k
set modulo near-ties, and the attention output and lse against the oracle's
attention over the oracle's own set (for rows whose GPU set differs at a
near-tie, several sets are correct: the GPU attention is re-run on the
oracle's set for them).

Sampled rows always include the first and last rows and the rows around the
point where the visible count crosses k."""
import numpy as np
import pytest
import torch

import bench
import oracle
from gpu_util import bf16_to_f32, check_attention, check_idx_sets, check_scores, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsa():
    import sparse_attention_16_amd as m
    assert torch.cuda.is_available()
    return m


def _rows(name, T, k, rng):
    base = {0, T - 1, T // 2}
    if name.startswith("prefill"):
        base |= {k - 2, k - 1, k, k + 1}
    extra = rng.choice(T, size=min(T, 10), replace=False)
    return np.array(sorted(r for r in base | set(int(x) for x in extra) if 0 <= r < T))


@pytest.mark.parametrize("name", ["prefill_4k", "decode_64k", "chunked_128k", "prefill_32k"])
def test_fullsize_sampled_rows(dsa, name):
    say(f"[fullsize] {name}")
    wl, entry = bench.make_workload(name)
    b = wl.batch
    d = wl.device("cuda")
    torch.cuda.synchronize()
    batch = dsa.Batch.from_host(b.cu_q, b.cu_kv, b.pos0)
    args = dsa.fwd_args(batch, d["qi"], d["qs"], d["w"], d["ki"], d["ks"], d["q"], d["kv"], wl.k,
                        wl.scale)
    out = torch.empty((b.T, 128, 512), dtype=torch.int16, device="cuda")
    lse = torch.empty((b.T, 128), device="cuda")
    idx = torch.empty((b.T, wl.k), dtype=torch.int32, device="cuda")
    fn = dsa.prefill_fwd if entry == "prefill" else dsa.decode_fwd
    fn(args, batch, out, lse, idx)
    torch.cuda.synchronize()
    say(f"  {name}: fused forward done (T={b.T}, max_kv={b.max_kv})")

    rng = np.random.default_rng(2024)
    rows = np.arange(b.T) if entry == "decode" else _rows(name, b.T, wl.k, rng)
    rsel = torch.as_tensor(rows, device="cuda")
    g_idx = idx[rsel].cpu().numpy()
    g_out = bf16_to_f32(out[rsel])
    g_lse = lse[rsel].cpu().numpy()

    # index scores of the same rows through the standalone indexer entry
    ld = ((b.max_kv + 63) // 64) * 64
    scores = torch.empty((b.T, ld), dtype=torch.float32, device="cuda")
    dsa.indexer_scores(batch, d["qi"], d["qs"], d["w"], d["ki"], d["ks"], scores)
    g_scores = scores[rsel].cpu().numpy()
    del scores
    torch.cuda.empty_cache()

    inp = wl.sampled_host(rows)
    ref_s, A = oracle.indexer(b.cu_q, b.cu_kv, b.pos0, inp.qi, inp.qi_scale, inp.w, inp.ki,
                              inp.ki_scale, rows=rows, ld=ld, want_abs=True)
    _, _, ctx, _, nvis = oracle.visible(b.cu_q, b.cu_kv, b.pos0)
    worst = check_scores(g_scores, ref_s, A, nvis[rows], name)
    say(f"  {name}: {len(rows)} rows, worst relative score error {worst:.3g}")

    ref_idx = oracle.topk(b.cu_q, b.cu_kv, b.pos0, ref_s, wl.k, rows=rows)
    differ = check_idx_sets(g_idx, ref_idx, ref_s, A, nvis[rows], wl.k, name)
    say(f"  {name}: {len(differ)} rows differ only at near-ties")
    assert len(differ) <= max(2, len(rows) // 10)
    # attention against the oracle over the oracle's own set; rows whose GPU
    # set differs at near-ties are recomputed by the GPU attention on that set
    same = np.setdiff1d(np.arange(len(rows)), differ)
    o_ref, l_ref = oracle.sparse_attn(b.cu_q, b.cu_kv, b.pos0, inp.q, inp.kv, ref_idx, wl.Dv,
                                      wl.scale, rows=rows)
    dl, rel = check_attention(g_out[same], g_lse[same], o_ref[same], l_ref[same], name)
    if differ:
        fix = idx.clone()
        fix[torch.as_tensor(rows[differ], device="cuda")] = torch.from_numpy(ref_idx[differ]).cuda()
        out2 = torch.empty_like(out)
        lse2 = torch.empty_like(lse)
        dsa.sparse_mla_fwd(batch, d["q"], d["kv"], fix, wl.scale, out2, lse2)
        sel = torch.as_tensor(rows[differ], device="cuda")
        check_attention(bf16_to_f32(out2[sel]), lse2[sel].cpu().numpy(), o_ref[differ], l_ref[differ],
                        name + " (oracle set)")
    say(f"  {name}: attention max |dlse| {dl:.3g}, max row ||do||/||o|| {rel:.3g}")
