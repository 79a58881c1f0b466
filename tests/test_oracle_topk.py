"""Pins for the oracle's top-k selection (section "Отбор и основное внимание"
of the DSA technical-report reading): the pairwise characterisation of the
selected set, numpy's stable argsort, exact ties, short rows, +-0."""
import numpy as np
import pytest

import oracle
import synth


def _one_row(scores, k):
    n = len(scores)
    b = synth.Batch.prefill(1, n, n - 1)
    return oracle.topk(b.cu_q, b.cu_kv, b.pos0, np.asarray(scores, np.float32)[None, :], k)[0]


def _dominates(scores, sel):
    """The selected set is the unique set where every member beats every
    non-member: larger score, or equal score and lower position."""
    sset = set(int(s) for s in sel if s >= 0)
    others = [s for s in range(len(scores)) if s not in sset]
    for a in sset:
        for o in others:
            va, vo = np.float32(scores[a]), np.float32(scores[o])
            if not (va > vo or (va == vo and a < o)):
                return False
    return True


@pytest.mark.parametrize("seed", range(6))
def test_pairwise_characterisation_small(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 40))
    k = int(rng.integers(1, 12))
    # few distinct values -> many exact ties
    scores = rng.integers(-3, 4, size=n).astype(np.float32)
    sel = _one_row(scores, k)
    m = min(n, k)
    assert np.all(sel[m:] == -1)
    got = sel[:m]
    assert np.all(np.diff(got) > 0)  # ascending, no duplicates
    assert _dominates(scores, got)


def test_matches_stable_argsort():
    rng = np.random.default_rng(7)
    for n, k in [(100, 10), (1000, 64), (5000, 2048), (3000, 2048), (2048, 2048)]:
        scores = rng.standard_normal(n).astype(np.float32)
        scores[rng.integers(0, n, size=n // 10)] = 0.5  # a block of exact ties
        sel = _one_row(scores, k)
        ref = np.sort(np.argsort(-scores, kind="stable")[:min(n, k)])
        assert np.array_equal(sel[:min(n, k)], ref)
        assert np.all(sel[min(n, k):] == -1)


def test_short_row_selects_everything():
    scores = np.array([3.0, -1.0, np.float32(-1e30), 2.0], np.float32)
    assert _one_row(scores, 8).tolist() == [0, 1, 2, 3, -1, -1, -1, -1]


def test_signed_zero_is_a_tie():
    scores = np.array([1.0, -0.0, 0.0, -0.0, -1.0], np.float32)
    assert _one_row(scores, 2).tolist() == [0, 1]
    scores = np.array([1.0, 0.0, -0.0, -1.0], np.float32)
    assert _one_row(scores, 2).tolist() == [0, 1]


def test_duplicate_keys_tie_to_lower_index():
    # duplicated key rows give bit-identical scores; the lower position wins
    inp = synth.make_inputs(synth.Batch.prefill(1, 300, 299), seed=31, HI=4, DI=32, H=2, D=16, Dv=8)
    ki = inp.ki.copy()
    ks = inp.ki_scale.copy()
    for a, bb in [(10, 250), (20, 270), (33, 299)]:
        ki[bb] = ki[a]
        ks[bb] = ks[a]
    b = inp.batch
    s = oracle.indexer(b.cu_q, b.cu_kv, b.pos0, inp.qi, inp.qi_scale, inp.w, ki, ks)
    assert s[0, 10] == s[0, 250] and s[0, 33] == s[0, 299]
    order = np.argsort(-s[0], kind="stable")
    for kk in range(1, 300):
        sel = oracle.topk(b.cu_q, b.cu_kv, b.pos0, s, kk)[0]
        assert np.array_equal(sel, np.sort(order[:kk]))
        assert _dominates(s[0], sel)


def test_causal_rows_only_see_visible_keys():
    inp = synth.make_inputs(synth.Batch.prefill(50, 50, 0), seed=32, HI=4, DI=32, H=2, D=16, Dv=8)
    b = inp.batch
    s = oracle.indexer(b.cu_q, b.cu_kv, b.pos0, inp.qi, inp.qi_scale, inp.w, inp.ki, inp.ki_scale)
    idx = oracle.topk(b.cu_q, b.cu_kv, b.pos0, s, 16)
    for t in range(50):
        sel = idx[t][idx[t] >= 0]
        assert len(sel) == min(t + 1, 16)
        assert sel.max() <= t
        if t + 1 <= 16:
            assert sel.tolist() == list(range(t + 1))


def test_min_selected_at_least_max_unselected():
    inp = synth.make_inputs(synth.Batch.prefill(8, 600, 592), seed=33, HI=8, DI=32, H=2, D=16, Dv=8)
    b = inp.batch
    s = oracle.indexer(b.cu_q, b.cu_kv, b.pos0, inp.qi, inp.qi_scale, inp.w, inp.ki, inp.ki_scale)
    idx = oracle.topk(b.cu_q, b.cu_kv, b.pos0, s, 100)
    for t in range(8):
        n = 593 + t
        mask = np.zeros(n, bool)
        mask[idx[t]] = True
        assert s[t, :n][mask].min() >= s[t, :n][~mask].max()
