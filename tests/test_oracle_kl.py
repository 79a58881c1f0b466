"""Pins for the oracle's indexer KL loss (page "Техотчёт DeepSeek-V3.2 (2025):
разреженное внимание DSA и масштабирование RL", section "Как учили
индексатор": the target is the main attention summed over heads and
L1-normalised over the key set, the loss is KL(target || softmax of the index
scores), over every visible key in the dense warm-up and over the selected
keys in the sparse stage).

Each pin ties the oracle to something other than itself:
  * one head: the target is one softmax, and the loss is torch's library
    KL divergence (torch.nn.functional.kl_div) between two softmaxes;
  * two heads of different logit scale: the target is the mean of the two
    heads' library softmaxes (torch.softmax), each normalised on its own;
  * all heads equal: the head sum normalised is that same softmax, so index
    scores equal to the logits give zero loss, and doubled logits give the
    library KL;
  * zero queries: the target is uniform, KL(U || r) = ln-sum-exp(I) - mean(I) - ln m;
  * invariances: a constant added to I, the order of the slots, the order of
    the heads, -1 slots;
  * dense == sparse over all visible keys; p sums to 1; KL >= 0.
"""
import numpy as np
import torch

import oracle
import synth


def _small(T=6, N=9, H=4, D=8, seed=0):
    rng = np.random.default_rng(seed)
    b = synth.Batch.prefill(T, N, N - T)
    q = rng.standard_normal((T, H, D)).astype(np.float32)
    kv = rng.standard_normal((N, D)).astype(np.float32)
    scores = (rng.standard_normal((T, N)) * 2).astype(np.float32)
    return b, q, kv, scores


def _torch_kl(p_logits, i_scores):
    """KL(softmax(p_logits) || softmax(i_scores)) with torch's library KL."""
    lp = torch.log_softmax(torch.as_tensor(i_scores, dtype=torch.float64), dim=-1)
    tgt = torch.softmax(torch.as_tensor(p_logits, dtype=torch.float64), dim=-1)
    return float(torch.nn.functional.kl_div(lp, tgt, reduction="sum"))


def test_single_head_is_library_kl():
    b, q, kv, scores = _small(H=1, seed=1)
    scale = 0.37
    kl = oracle.indexer_kl(b.cu_q, b.cu_kv, b.pos0, q, kv, scale, scores)
    _, _, _, _, nvis = oracle.visible(b.cu_q, b.cu_kv, b.pos0)
    for t in range(b.T):
        n = int(nvis[t])
        z = scale * (kv[:n].astype(np.float64) @ q[t, 0].astype(np.float64))
        assert abs(kl[t] - _torch_kl(z, scores[t, :n])) < 1e-12


def test_equal_heads_reduce_to_one_softmax():
    b, q, kv, scores = _small(H=5, seed=2)
    q[:] = q[:, :1, :]                          # every head the same query
    scale = 0.5
    _, _, _, _, nvis = oracle.visible(b.cu_q, b.cu_kv, b.pos0)
    z = np.zeros_like(scores)
    for t in range(b.T):
        n = int(nvis[t])
        z[t, :n] = scale * (kv[:n].astype(np.float64) @ q[t, 0].astype(np.float64))
    # index scores equal to the (float32-rounded) logits: loss within rounding of 0
    kl0 = oracle.indexer_kl(b.cu_q, b.cu_kv, b.pos0, q, kv, scale, z)
    assert np.all(np.abs(kl0) < 1e-6)
    kl2 = oracle.indexer_kl(b.cu_q, b.cu_kv, b.pos0, q, kv, scale, 2 * z)
    for t in range(b.T):
        n = int(nvis[t])
        zz = scale * (kv[:n].astype(np.float64) @ q[t, 0].astype(np.float64))
        assert abs(kl2[t] - _torch_kl(zz, (2 * z[t, :n]).astype(np.float32))) < 1e-9


def test_two_heads_target_is_mean_of_softmaxes():
    # heads with very different logit scales: each head's softmax is
    # normalised before the sum (a sum of exp without per-head normalisation,
    # or a softmax of the summed logits, gives a different target)
    b, q, kv, scores = _small(H=2, seed=7)
    q[:, 1, :] *= 6.0
    scale = 0.45
    kl, p = oracle.indexer_kl(b.cu_q, b.cu_kv, b.pos0, q, kv, scale, scores, want_p=True)
    _, _, _, _, nvis = oracle.visible(b.cu_q, b.cu_kv, b.pos0)
    for t in range(b.T):
        n = int(nvis[t])
        z = scale * torch.as_tensor(kv[:n], dtype=torch.float64) @ torch.as_tensor(q[t], dtype=torch.float64).T
        tgt = 0.5 * (torch.softmax(z[:, 0], 0) + torch.softmax(z[:, 1], 0))
        assert np.allclose(p[t, :n], tgt.numpy(), rtol=1e-12, atol=1e-15)
        lp = torch.log_softmax(torch.as_tensor(scores[t, :n], dtype=torch.float64), 0)
        assert abs(kl[t] - float(torch.nn.functional.kl_div(lp, tgt, reduction="sum"))) < 1e-12


def test_zero_queries_uniform_target_closed_form():
    b, q, kv, scores = _small(H=3, seed=3)
    q[:] = 0.0
    kl, p = oracle.indexer_kl(b.cu_q, b.cu_kv, b.pos0, q, kv, 1.0, scores, want_p=True)
    _, _, _, _, nvis = oracle.visible(b.cu_q, b.cu_kv, b.pos0)
    for t in range(b.T):
        n = int(nvis[t])
        s = scores[t, :n].astype(np.float64)
        lse = s.max() + np.log(np.sum(np.exp(s - s.max())))
        assert abs(kl[t] - (lse - s.mean() - np.log(n))) < 1e-12
        assert np.allclose(p[t, :n], 1.0 / n, rtol=0, atol=1e-15)


def test_invariances_and_positivity():
    b, q, kv, scores = _small(T=5, N=12, H=4, seed=4)
    base, p = oracle.indexer_kl(b.cu_q, b.cu_kv, b.pos0, q, kv, 0.3, scores, want_p=True)
    assert np.all(base >= 0)
    _, _, _, _, nvis = oracle.visible(b.cu_q, b.cu_kv, b.pos0)
    for t in range(b.T):
        assert abs(np.sum(p[t, :int(nvis[t])]) - 1.0) < 1e-12
    shifted = oracle.indexer_kl(b.cu_q, b.cu_kv, b.pos0, q, kv, 0.3, scores + np.float32(4.0))
    assert np.allclose(shifted, base, rtol=1e-6, atol=1e-9)
    heads = oracle.indexer_kl(b.cu_q, b.cu_kv, b.pos0, q[:, ::-1, :].copy(), kv, 0.3, scores)
    assert np.allclose(heads, base, rtol=1e-12, atol=1e-14)


def test_sparse_over_all_visible_equals_dense_and_ignores_order_and_padding():
    b, q, kv, scores = _small(T=6, N=10, H=3, seed=5)
    dense, pd = oracle.indexer_kl(b.cu_q, b.cu_kv, b.pos0, q, kv, 0.4, scores, want_p=True)
    _, _, _, _, nvis = oracle.visible(b.cu_q, b.cu_kv, b.pos0)
    k = 13
    rng = np.random.default_rng(0)
    idx = np.full((b.T, k), -1, np.int32)
    for t in range(b.T):
        n = int(nvis[t])
        slots = rng.permutation(k)[:n]          # visible keys scattered among -1 slots
        idx[t, slots] = rng.permutation(n)
    sparse, ps = oracle.indexer_kl(b.cu_q, b.cu_kv, b.pos0, q, kv, 0.4, scores, idx=idx, want_p=True)
    assert np.allclose(sparse, dense, rtol=1e-12, atol=1e-14)
    for t in range(b.T):
        valid = idx[t] >= 0
        assert np.allclose(ps[t, valid], pd[t, idx[t, valid]], rtol=1e-12, atol=1e-15)
        assert np.all(ps[t, ~valid] == 0.0)


def test_single_key_and_empty_rows():
    b = synth.Batch.ragged([2, 1], [1, 0], [0, 0])   # one key; then a sequence with no cache
    rng = np.random.default_rng(6)
    q = rng.standard_normal((3, 2, 4)).astype(np.float32)
    kv = rng.standard_normal((1, 4)).astype(np.float32)
    scores = rng.standard_normal((3, 1)).astype(np.float32)
    kl = oracle.indexer_kl(b.cu_q, b.cu_kv, b.pos0, q, kv, 1.0, scores)
    assert np.all(kl == 0.0)
