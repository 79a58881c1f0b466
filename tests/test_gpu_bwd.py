"""GPU parity of the sparse attention backward (dsa_sparse_mla_bwd) against the
oracle's exact backward (page "Техотчёт DeepSeek-V3.2 (2025): разреженное
внимание DSA и масштабирование RL": the attention of section "Отбор и основное
внимание", trained in the sparse stage of section "Как учили индексатор").

Every input of the GPU call comes from the input generator or the oracle: q
and the latent cache (generator), the selection (oracle top-k, or hand-made
with holes and repeats), the forward's out and lse (oracle attention, out
rounded to bf16 as the forward returns it), dout (seeded normals in bf16).
The backward's contract takes delta = <dout, out> from the out it is handed
(a bf16 output moves dq by -scale * d(delta) * sum_j P kv_j, up to 1e-2 on rows
with few keys), so the oracle is given the same out.

Tolerance: the GPU rounds P and dZ to bf16 (relative 2^-9) before the products
that consume them and takes delta from the bf16 forward output, so its errors
are of order 2e-3 of a row's typical magnitude; the gate per (row, head) of dq
and per cache row of dkv is |d| <= 3e-2 * rms(ref row) + 1e-2 * |ref|.  The
worst error relative to the row RMS is printed.  A row whose exact gradient
is 0 (a single selected key: the softmax has no gradient) is held to an
absolute floor of 1e-4 times the whole tensor's RMS (fp32 rounding of
dP - delta leaves ~1e-7 there).
"""
import numpy as np
import pytest
import torch

import bench
import oracle
import synth
from gpu_util import dev, say

pytestmark = pytest.mark.gpu

RMS_TOL, REL_TOL = 3e-2, 1e-2
ABS_FLOOR = 1e-4    # x the whole tensor's rms: rows whose exact gradient is 0 (one selected key)


@pytest.fixture(scope="module")
def dsa():
    import sparse_attention_16_amd as m  # fails loudly when libdsa.so is missing
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def _bf16_bits(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy() \
        .view(np.uint16)


def _check_rows(got, ref, what):
    """got/ref [rows, n] (one gradient row per line)."""
    rms = np.sqrt(np.mean(ref ** 2, axis=1, keepdims=True))
    floor = ABS_FLOOR * np.sqrt(np.mean(ref ** 2)) if ref.size else 0.0
    err = np.abs(got.astype(np.float64) - ref)
    bad = err > RMS_TOL * rms + REL_TOL * np.abs(ref) + floor
    assert not np.any(bad), f"{what}: {bad.sum()} values out of tolerance, worst {err.max():.3g}"
    live = rms[:, 0] > 0                      # (rows with an exact zero gradient are held to the floor)
    rel = err[live] / rms[live]
    return float(rel.max()) if rel.size else 0.0


def _inputs(inp, idx, seed):
    b = inp.batch
    o, lse = oracle.sparse_attn(b.cu_q, b.cu_kv, b.pos0, inp.q, inp.kv, idx, inp.Dv, inp.scale)
    rng = np.random.default_rng(seed)
    dout = _bf16_bits(rng.standard_normal((b.T, inp.H, inp.Dv)))
    return _bf16_bits(o), lse, dout


def _run(dsa, inp, idx, out, lse, dout):
    b = inp.batch
    batch = dsa.Batch.from_host(b.cu_q, b.cu_kv, b.pos0)
    dq = torch.empty((b.T, inp.H, inp.D), dtype=torch.float32, device="cuda")
    dkv = torch.full((b.N, inp.D), float("nan"), dtype=torch.float32, device="cuda")
    dsa.sparse_mla_bwd(batch, dev(inp.q), dev(inp.kv), dev(idx), inp.scale, dev(out), dev(lse), dev(dout), dq, dkv)
    torch.cuda.synchronize()
    return dq.cpu().numpy(), dkv.cpu().numpy()


def _compare(dsa, inp, idx, seed, what):
    b = inp.batch
    out, lse, dout = _inputs(inp, idx, seed)
    dq_ref, dkv_ref = oracle.sparse_attn_bwd(b.cu_q, b.cu_kv, b.pos0, inp.q, inp.kv, dout, idx, inp.Dv, inp.scale,
                                             out=out)
    dq, dkv = _run(dsa, inp, idx, out, lse, dout)
    e_q = _check_rows(dq.reshape(-1, inp.D), dq_ref.reshape(-1, inp.D), what + " dq")
    touched = np.any(dkv_ref != 0, axis=1)
    e_kv = _check_rows(dkv[touched], dkv_ref[touched], what + " dkv")
    assert np.all(dkv[~touched] == 0.0), f"{what}: dkv rows no slot selects must be zero"
    say(f"  {what}: worst error / row rms: dq {e_q:.3g}, dkv {e_kv:.3g}")


CASES = {
    "prefill_300_k64": lambda: synth.make_inputs(synth.Batch.prefill(300, 300, 0), seed=181, k=64),
    "prefill_700_k256": lambda: synth.make_inputs(synth.Batch.prefill(700, 700, 0), seed=182, k=256),
    "ragged_k100": lambda: synth.make_inputs(synth.Batch.ragged([70, 1, 33, 2], [200, 90, 33, 0], [130, 89, 0, 0]),
                                             seed=183, k=100),
    "decode_k2048": lambda: synth.make_inputs(synth.Batch.decode([1, 40, 2049, 9000]), seed=184, k=2048,
                                              per_seq=True),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_sparse_mla_bwd_matches_oracle(dsa, name):
    say(f"[sparse_mla_bwd] {name}")
    inp = CASES[name]()
    b = inp.batch
    scores = oracle.indexer(b.cu_q, b.cu_kv, b.pos0, inp.qi, inp.qi_scale, inp.w, inp.ki, inp.ki_scale)
    idx = oracle.topk(b.cu_q, b.cu_kv, b.pos0, scores, inp.k)
    _compare(dsa, inp, idx, 1000 + len(name), name)


def test_sparse_mla_bwd_holes_repeats_and_empty_rows(dsa):
    inp = synth.make_inputs(synth.Batch.prefill(48, 3000, 2952), seed=185, k=300)
    rng = np.random.default_rng(12)
    idx = np.full((48, 300), -1, np.int32)
    for t in range(48):
        n = [0, 1, 31, 32, 33, 299, 300, 150][t % 8]
        idx[t, :n] = rng.choice(2953 + t, n, replace=False)
    idx[rng.random(idx.shape) < 0.1] = -1
    idx[9, :20] = 17                            # one row listed 20 times: its gradient counts 20 slots
    idx[13, 5:9] = idx[14, 5:9] = 1000          # the same row from several query rows
    _compare(dsa, inp, idx, 77, "holes")


def test_sparse_mla_bwd_32k_sampled(dsa):
    """The 32K-prefill backward bench.py times (sparse_bwd_32k): every row
    runs; dout is zero except on sampled rows, so dkv holds exactly their
    contributions and every other row's dq is exactly 0."""
    say("[fullsize] sparse_bwd_32k")
    wl, _ = bench.make_workload("prefill_32k")
    b = wl.batch
    d = wl.device("cuda")
    rows = np.array([0, 1, 2047, 2048, 2049, 16000, 32767])
    inp = wl.sampled_host(rows)
    ld = ((b.max_kv + 63) // 64) * 64
    s_rows = oracle.indexer(b.cu_q, b.cu_kv, b.pos0, inp.qi, inp.qi_scale, inp.w, inp.ki, inp.ki_scale, rows=rows,
                            ld=ld)
    idx_rows = oracle.topk(b.cu_q, b.cu_kv, b.pos0, s_rows, wl.k, rows=rows)
    o_rows, lse_rows = oracle.sparse_attn(b.cu_q, b.cu_kv, b.pos0, inp.q, inp.kv, idx_rows, wl.Dv, wl.scale,
                                          rows=rows)
    rng = np.random.default_rng(5)
    dout_rows = _bf16_bits(rng.standard_normal((len(rows), 128, wl.Dv)))
    dout_full = np.zeros((b.T, 128, wl.Dv), np.uint16)
    dout_full[rows] = dout_rows
    out_full = np.zeros((b.T, 128, wl.Dv), np.uint16)
    out_full[rows] = _bf16_bits(o_rows)
    dq_ref, dkv_ref = oracle.sparse_attn_bwd(b.cu_q, b.cu_kv, b.pos0, inp.q, inp.kv, dout_full, idx_rows, wl.Dv,
                                             wl.scale, rows=rows, out=out_full)
    # full-size inputs: the sampled rows from the oracle, the others a valid filler
    idx = torch.full((b.T, wl.k), -1, dtype=torch.int32, device="cuda")
    idx[:, 0] = 0
    out = torch.zeros((b.T, 128, wl.Dv), dtype=torch.int16, device="cuda")
    lse = torch.zeros((b.T, 128), dtype=torch.float32, device="cuda")
    dout = torch.zeros((b.T, 128, wl.Dv), dtype=torch.int16, device="cuda")
    r = torch.as_tensor(rows, device="cuda")
    idx[r] = dev(idx_rows)
    out[r] = dev(_bf16_bits(o_rows))
    lse[r] = dev(lse_rows)
    dout[r] = dev(dout_rows)
    batch = dsa.Batch.from_host(b.cu_q, b.cu_kv, b.pos0)
    dq = torch.empty((b.T, 128, 576), dtype=torch.float32, device="cuda")
    dkv = torch.empty((b.N, 576), dtype=torch.float32, device="cuda")
    dsa.sparse_mla_bwd(batch, d["q"], d["kv"], idx, wl.scale, out, lse, dout, dq, dkv)
    torch.cuda.synchronize()
    e_q = _check_rows(dq[r].cpu().numpy().reshape(-1, 576), dq_ref.reshape(-1, 576), "32k dq")
    others = torch.ones(b.T, dtype=torch.bool, device="cuda")
    others[r] = False
    assert float(dq[others].abs().max()) == 0.0
    g = dkv.cpu().numpy()
    touched = np.any(dkv_ref != 0, axis=1)
    e_kv = _check_rows(g[touched], dkv_ref[touched], "32k dkv")
    assert np.all(g[~touched] == 0.0)
    say(f"  32k: worst error / row rms: dq {e_q:.3g}, dkv {e_kv:.3g}")


@pytest.mark.parametrize("name", ["prefill_300_k64", "decode_k2048"])
def test_sparse_mla_bwd_against_exact_gradient(dsa, name):
    """The GPU backward (handed the forward's bf16 out, as in training) against
    the oracle's exact gradient, whose delta comes from the exact forward
    output.  Bound: the rounding gate above plus the closed-form shift that the
    bf16 out causes, -scale * (delta(out_bf16) - delta(exact)) * sum_j P_j kv_j
    in dq (and its image in dkv), which the oracle evaluates as the difference
    of its two gradients (delta from the bf16 out minus delta exact)."""
    say(f"[sparse_mla_bwd exact] {name}")
    inp = CASES[name]()
    b = inp.batch
    scores = oracle.indexer(b.cu_q, b.cu_kv, b.pos0, inp.qi, inp.qi_scale, inp.w, inp.ki, inp.ki_scale)
    idx = oracle.topk(b.cu_q, b.cu_kv, b.pos0, scores, inp.k)
    out, lse, dout = _inputs(inp, idx, 2000 + len(name))
    args = (b.cu_q, b.cu_kv, b.pos0, inp.q, inp.kv, dout, idx, inp.Dv, inp.scale)
    dq_ex, dkv_ex = oracle.sparse_attn_bwd(*args)
    dq_bf, dkv_bf = oracle.sparse_attn_bwd(*args, out=out)
    dq, dkv = _run(dsa, inp, idx, out, lse, dout)

    def check(got, exact, shifted, what):
        got, exact, shifted = (x.reshape(x.shape[0], -1).astype(np.float64) for x in (got, exact, shifted))
        rms = np.sqrt(np.mean(exact ** 2, axis=1, keepdims=True))
        floor = ABS_FLOOR * np.sqrt(np.mean(exact ** 2))
        shift = np.abs(shifted - exact)
        err = np.abs(got - exact)
        bad = err > RMS_TOL * rms + REL_TOL * np.abs(exact) + shift + floor
        assert not np.any(bad), f"{name} {what}: {bad.sum()} values outside the bound, worst {err.max():.3g}"
        live = rms[:, 0] > 0
        return float(np.max(err[live] / rms[live])), float(np.max(shift[live] / rms[live]))

    e_q, s_q = check(dq.reshape(-1, inp.D), dq_ex.reshape(-1, inp.D), dq_bf.reshape(-1, inp.D), "dq")
    touched = np.any(dkv_ex != 0, axis=1)
    e_kv, s_kv = check(dkv[touched], dkv_ex[touched], dkv_bf[touched], "dkv")
    assert np.all(dkv[~touched] == 0.0)
    say(f"  {name}: worst error / row rms against the exact gradient: dq {e_q:.3g} (bf16-out shift {s_q:.3g}), "
        f"dkv {e_kv:.3g} (shift {s_kv:.3g})")
