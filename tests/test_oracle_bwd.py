"""Pins for the oracle's backward of the sparse MQA attention (the attention
of page "Техотчёт DeepSeek-V3.2 (2025): разреженное внимание DSA и
масштабирование RL", section "Отбор и основное внимание", differentiated for
the sparse training stage of section "Как учили индексатор").

Each pin ties the hand-derived backward to something other than itself:
  * torch autograd (float64) of the same forward written with library ops
    (index_select, matmul, softmax): an independent derivation of every
    gradient, including repeated and -1 slots;
  * central finite differences of the oracle's own forward attention;
  * one selected key: the softmax has zero gradient, so dq = 0 and dkv is
    sum_h dout[h] in the value dims, 0 in the rest;
  * identical key rows: dq = 0 (the softmax's gradient sums to 0 per head);
  * linearity in dout;
  * delta from a given forward output: the exact output reproduces the exact
    delta, and a perturbation moves dq by the closed-form amount.
"""
import numpy as np
import torch

import oracle
import synth


def _case(T=5, N=11, H=3, D=6, Dv=4, k=7, seed=0):
    rng = np.random.default_rng(seed)
    b = synth.Batch.prefill(T, N, N - T)
    q = rng.standard_normal((T, H, D)).astype(np.float32)
    kv = rng.standard_normal((N, D)).astype(np.float32)
    dout = rng.standard_normal((T, H, Dv)).astype(np.float32)
    idx = np.full((T, k), -1, np.int32)
    for t in range(T):
        n = rng.integers(1, k + 1)
        idx[t, :n] = rng.integers(0, N - T + t + 1, n)      # repeats allowed, all visible
    return b, q, kv, dout, idx


def _torch_grads(b, q, kv, dout, idx, Dv, scale):
    qt = torch.tensor(q, dtype=torch.float64, requires_grad=True)
    kvt = torch.tensor(kv, dtype=torch.float64, requires_grad=True)
    loss = torch.zeros((), dtype=torch.float64)
    for t in range(q.shape[0]):
        sel = torch.as_tensor(idx[t][idx[t] >= 0], dtype=torch.long)   # one sequence: positions are rows
        rows = kvt.index_select(0, sel)                                 # [m, D]
        z = scale * qt[t] @ rows.T                                      # [H, m]
        o = torch.softmax(z, dim=-1) @ rows[:, :Dv]                     # [H, Dv]
        loss = loss + (torch.as_tensor(dout[t], dtype=torch.float64) * o).sum()
    loss.backward()
    return qt.grad.numpy(), kvt.grad.numpy()


def test_matches_torch_autograd():
    b, q, kv, dout, idx = _case(seed=1)
    scale = 0.35
    dq, dkv = oracle.sparse_attn_bwd(b.cu_q, b.cu_kv, b.pos0, q, kv, dout, idx, 4, scale)
    gq, gkv = _torch_grads(b, q, kv, dout, idx, 4, scale)
    assert np.allclose(dq, gq, rtol=1e-10, atol=1e-12)
    assert np.allclose(dkv, gkv, rtol=1e-10, atol=1e-12)


def test_finite_differences_of_the_oracle_forward():
    b, q, kv, dout, idx = _case(T=3, N=7, H=2, D=4, Dv=3, k=5, seed=2)
    scale = 0.5
    dq, dkv = oracle.sparse_attn_bwd(b.cu_q, b.cu_kv, b.pos0, q, kv, dout, idx, 3, scale)

    def loss(qq, kk):
        o, _ = oracle.sparse_attn(b.cu_q, b.cu_kv, b.pos0, qq, kk, idx, 3, scale)
        return float(np.sum(o.astype(np.float64) * dout))
    h = 1e-2
    for (t, hh, d) in [(0, 0, 0), (1, 1, 3), (2, 0, 2)]:
        qp, qm = q.copy(), q.copy()
        qp[t, hh, d] += h
        qm[t, hh, d] -= h
        fd = (loss(qp, kv) - loss(qm, kv)) / (2 * h)
        assert abs(fd - dq[t, hh, d]) < 2e-3 * max(1.0, abs(dq[t, hh, d]))
    for (s, d) in [(1, 0), (4, 2), (5, 3), (6, 1)]:
        kp, km = kv.copy(), kv.copy()
        kp[s, d] += h
        km[s, d] -= h
        fd = (loss(q, kp) - loss(q, km)) / (2 * h)
        assert abs(fd - dkv[s, d]) < 2e-3 * max(1.0, abs(dkv[s, d]))


def test_single_key_closed_form():
    b, q, kv, dout, idx = _case(seed=3)
    idx[:] = -1
    idx[:, 2] = np.arange(5)                       # one key per row (positions 0..4, all visible)
    dq, dkv = oracle.sparse_attn_bwd(b.cu_q, b.cu_kv, b.pos0, q, kv, dout, idx, 4, 0.7)
    assert np.all(np.abs(dq) < 1e-12)
    want = np.zeros_like(dkv)
    for t in range(5):
        want[t, :4] += dout[t].astype(np.float64).sum(axis=0)
    assert np.allclose(dkv, want, rtol=1e-12, atol=1e-12)


def test_identical_keys_give_zero_query_gradient_and_linearity():
    b, q, kv, dout, idx = _case(seed=4)
    kv[:] = kv[0]
    dq, dkv = oracle.sparse_attn_bwd(b.cu_q, b.cu_kv, b.pos0, q, kv, dout, idx, 4, 0.4)
    assert np.all(np.abs(dq) < 1e-12)
    b, q, kv, dout, idx = _case(seed=5)
    dq1, dkv1 = oracle.sparse_attn_bwd(b.cu_q, b.cu_kv, b.pos0, q, kv, dout, idx, 4, 0.4)
    dq2, dkv2 = oracle.sparse_attn_bwd(b.cu_q, b.cu_kv, b.pos0, q, kv, 2 * dout, idx, 4, 0.4)   # exact in f32
    assert np.allclose(dq2, 2 * dq1, rtol=1e-12, atol=1e-14)
    assert np.allclose(dkv2, 2 * dkv1, rtol=1e-12, atol=1e-14)


def test_delta_from_a_given_forward_output():
    # delta taken from the forward's own output (in double, as it returns it in
    # f32) matches the exact one; a perturbed output moves dq by exactly
    # -scale * d(delta)_h * sum_j P[j,h] kv[s_j,:]
    b, q, kv, dout, idx = _case(seed=6)
    scale = 0.45
    o, _ = oracle.sparse_attn(b.cu_q, b.cu_kv, b.pos0, q, kv, idx, 4, scale)
    dq0, dkv0 = oracle.sparse_attn_bwd(b.cu_q, b.cu_kv, b.pos0, q, kv, dout, idx, 4, scale)
    dq1, dkv1 = oracle.sparse_attn_bwd(b.cu_q, b.cu_kv, b.pos0, q, kv, dout, idx, 4, scale, out=o)
    assert np.allclose(dq1, dq0, rtol=1e-5, atol=1e-6) and np.allclose(dkv1, dkv0, rtol=1e-5, atol=1e-6)
    o2 = o.copy()
    o2[2, 1, :] += np.float32(0.25)
    dq2, _ = oracle.sparse_attn_bwd(b.cu_q, b.cu_kv, b.pos0, q, kv, dout, idx, 4, scale, out=o2)
    ddelta = 0.25 * float(np.sum(dout[2, 1].astype(np.float64)))
    o_full, _ = oracle.sparse_attn(b.cu_q, b.cu_kv, b.pos0, q, kv, idx, 6, scale)   # sum_j P kv over all 6 dims
    assert np.allclose(dq2[2, 1] - dq1[2, 1], -scale * ddelta * o_full[2, 1].astype(np.float64), rtol=1e-4,
                       atol=1e-6)
    assert np.allclose(np.delete(dq2.reshape(-1, 6), 2 * 3 + 1, axis=0), np.delete(dq1.reshape(-1, 6), 2 * 3 + 1,
                                                                                     axis=0), rtol=0, atol=0)
