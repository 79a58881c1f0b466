"""Pins for the oracle's MQA-mode attention over selected latent rows (eq. u of
the DSA technical-report reading, section "Отбор и основное внимание"):
torch's scaled-dot-product attention in fp64 on the same mask, closed forms
(uniform weights, a single key), and invariants (k >= visible keys gives
dense attention, lse monotone in the selected set, convexity, permutation and
future independence)."""
import math

import numpy as np
import torch

import oracle
import synth


def _small(L=40, H=4, D=24, Dv=16, seed=41, n_kv=None, pos0=0):
    b = synth.Batch.prefill(L, n_kv or L, pos0)
    return synth.make_inputs(b, seed=seed, HI=4, DI=16, H=H, D=D, Dv=Dv, fp8=False)


def _f64(x):
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).double().numpy()
    return x.astype(np.float64)


def _sdpa_ref(inp, idx):
    """torch SDPA (fp64, CPU) with an additive mask: 0 on selected keys, -inf
    elsewhere; K and V are the same latent rows broadcast over heads."""
    b = inp.batch
    q = torch.from_numpy(_f64(inp.q))            # [T, H, D]
    kv = torch.from_numpy(_f64(inp.kv))          # [N, D]
    T, H, D = q.shape
    N = kv.shape[0]
    mask = torch.full((T, N), -math.inf, dtype=torch.float64)
    for t in range(T):
        for s in idx[t]:
            if s >= 0:
                mask[t, int(b.cu_kv[0]) + int(s)] = 0.0
    qh = q.permute(1, 0, 2).unsqueeze(0)                       # [1, H, T, D]
    kh = kv.unsqueeze(0).unsqueeze(0).expand(1, H, N, D)
    vh = kv[:, :inp.Dv].unsqueeze(0).unsqueeze(0).expand(1, H, N, inp.Dv)
    o = torch.nn.functional.scaled_dot_product_attention(
        qh, kh.contiguous(), vh.contiguous(), attn_mask=mask.unsqueeze(0).unsqueeze(0),
        scale=inp.scale)
    logits = inp.scale * (q.permute(1, 0, 2) @ kv.T) + mask.unsqueeze(0)  # [H, T, N]
    lse = torch.logsumexp(logits, dim=-1)
    return o[0].permute(1, 0, 2).numpy(), lse.permute(1, 0).numpy()


def _run(inp, idx):
    b = inp.batch
    return oracle.sparse_attn(b.cu_q, b.cu_kv, b.pos0, inp.q, inp.kv, idx, inp.Dv, inp.scale)


def test_matches_torch_sdpa_random_selection():
    inp = _small()
    rng = np.random.default_rng(0)
    k = 8
    idx = np.full((inp.batch.T, k), -1, np.int32)
    for t in range(inp.batch.T):
        m = min(t + 1, k)
        idx[t, :m] = np.sort(rng.choice(t + 1, size=m, replace=False))
    o, lse = _run(inp, idx)
    ro, rl = _sdpa_ref(inp, idx)
    assert np.allclose(o, ro, rtol=1e-6, atol=1e-6)
    assert np.allclose(lse, rl, rtol=1e-6, atol=1e-6)


def test_matches_torch_sdpa_bf16_inputs():
    b = synth.Batch.prefill(12, 30, 18)
    inp = synth.make_inputs(b, seed=42, HI=4, DI=16, H=3, D=40, Dv=32)
    rng = np.random.default_rng(1)
    idx = np.stack([np.sort(rng.choice(19 + t, size=10, replace=False)) for t in range(12)]).astype(np.int32)
    o, lse = _run(inp, idx)
    ro, rl = _sdpa_ref(inp, idx)
    assert np.allclose(o, ro, rtol=1e-6, atol=1e-6)
    assert np.allclose(lse, rl, rtol=1e-6, atol=1e-6)


def test_uniform_weights_closed_form():
    # q = 0: every selected key has logit 0 -> o = mean of the selected values, lse = ln m
    inp = _small(L=20)
    inp.q[:] = 0
    idx = np.full((20, 6), -1, np.int32)
    for t in range(20):
        m = min(t + 1, 4)
        idx[t, :m] = np.arange(t + 1 - m, t + 1)
    o, lse = _run(inp, idx)
    for t in range(20):
        sel = idx[t][idx[t] >= 0]
        mean = inp.kv[sel, :inp.Dv].astype(np.float64).mean(axis=0)
        assert np.allclose(o[t], mean[None, :], atol=1e-6)
        assert np.allclose(lse[t], math.log(len(sel)), atol=1e-6)


def test_single_key_and_k1():
    inp = _small(L=10)
    idx = np.full((10, 1), 0, np.int32)
    o, lse = _run(inp, idx)
    z0 = inp.scale * (inp.q.astype(np.float64) @ inp.kv[0].astype(np.float64))  # [T, H]
    assert np.allclose(o, np.broadcast_to(inp.kv[0, :inp.Dv], o.shape), atol=1e-7)
    assert np.allclose(lse, z0, atol=1e-6)


def test_empty_selection():
    inp = _small(L=4)
    idx = np.full((4, 3), -1, np.int32)
    o, lse = _run(inp, idx)
    assert np.all(o == 0) and np.all(np.isneginf(lse))


def test_sparse_equals_dense_when_k_covers_row():
    # tiny configuration with k = 256 >= every visible count: bitwise dense
    inp = synth.tiny_prefill(k=256)
    b = inp.batch
    s = oracle.indexer(b.cu_q, b.cu_kv, b.pos0, inp.qi, None, inp.w, inp.ki, None)
    idx = oracle.topk(b.cu_q, b.cu_kv, b.pos0, s, 256)
    o, lse = oracle.sparse_attn(b.cu_q, b.cu_kv, b.pos0, inp.q, inp.kv, idx, inp.Dv, inp.scale)
    do, dl = oracle.dense_attn(b.cu_q, b.cu_kv, b.pos0, inp.q, inp.kv, inp.Dv, inp.scale)
    assert np.array_equal(o, do) and np.array_equal(lse, dl)


def test_tiny_k32_sparse_properties():
    inp = synth.tiny_prefill(k=32)
    b = inp.batch
    s = oracle.indexer(b.cu_q, b.cu_kv, b.pos0, inp.qi, None, inp.w, inp.ki, None)
    idx = oracle.topk(b.cu_q, b.cu_kv, b.pos0, s, 32)
    o, lse = oracle.sparse_attn(b.cu_q, b.cu_kv, b.pos0, inp.q, inp.kv, idx, inp.Dv, inp.scale)
    do, dl = oracle.dense_attn(b.cu_q, b.cu_kv, b.pos0, inp.q, inp.kv, inp.Dv, inp.scale)
    # rows with at most 32 visible keys are dense; later rows attend to a subset
    assert np.array_equal(o[:32], do[:32]) and np.array_equal(lse[:32], dl[:32])
    assert np.all(lse[32:] <= dl[32:] + 1e-6)
    assert np.all(lse[33:] < dl[33:])
    # convexity: each output lies within the selected values' range
    for t in range(0, 256, 17):
        sel = idx[t][idx[t] >= 0]
        vals = inp.kv[sel, :inp.Dv]
        assert np.all(o[t] >= vals.min(axis=0) - 1e-5) and np.all(o[t] <= vals.max(axis=0) + 1e-5)


def test_dense_matches_sdpa_causal():
    inp = _small(L=24)
    idx = np.full((24, 24), -1, np.int32)
    for t in range(24):
        idx[t, :t + 1] = np.arange(t + 1)
    b = inp.batch
    do, dl = oracle.dense_attn(b.cu_q, b.cu_kv, b.pos0, inp.q, inp.kv, inp.Dv, inp.scale)
    ro, rl = _sdpa_ref(inp, idx)
    assert np.allclose(do, ro, rtol=1e-6, atol=1e-6) and np.allclose(dl, rl, rtol=1e-6, atol=1e-6)


def test_permutation_and_future_independence():
    inp = _small(L=30)
    rng = np.random.default_rng(5)
    idx = np.stack([np.sort(rng.choice(t + 1, size=min(t + 1, 7), replace=False)).tolist()
                    + [-1] * (7 - min(t + 1, 7)) for t in range(30)]).astype(np.int32)
    o, lse = _run(inp, idx)
    perm = idx[:, ::-1].copy()
    o2, lse2 = _run(inp, perm)
    assert np.allclose(o, o2, atol=1e-6) and np.allclose(lse, lse2, atol=1e-6)
    kv2 = inp.kv.copy()
    kv2[20:] = 7.0
    b = inp.batch
    o3, lse3 = oracle.sparse_attn(b.cu_q, b.cu_kv, b.pos0, inp.q, kv2, idx, inp.Dv, inp.scale)
    assert np.array_equal(o[:20], o3[:20]) and np.array_equal(lse[:20], lse3[:20])


def test_value_is_first_dv_dims():
    # changing only the rope dims (>= Dv) changes weights but not the value rows used
    inp = _small(L=6, D=24, Dv=16)
    inp.q[:] = 0  # logits all zero -> rope dims have no effect at all
    idx = np.tile(np.arange(6, dtype=np.int32), (6, 1))
    idx[np.arange(6)[:, None] < np.arange(6)[None, :]] = -1
    o, _ = _run(inp, idx)
    kv2 = inp.kv.copy()
    kv2[:, 16:] = 100.0
    b = inp.batch
    o2, _ = oracle.sparse_attn(b.cu_q, b.cu_kv, b.pos0, inp.q, kv2, idx, inp.Dv, inp.scale)
    assert np.array_equal(o, o2)
    kv3 = inp.kv.copy()
    kv3[:, :16] += 1.0
    o3, _ = oracle.sparse_attn(b.cu_q, b.cu_kv, b.pos0, inp.q, kv3, idx, inp.Dv, inp.scale)
    assert np.allclose(o3, o + 1.0, atol=1e-6)
