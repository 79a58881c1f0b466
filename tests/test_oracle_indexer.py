"""Pins for the oracle's index score (eq. I of the DSA technical-report reading,
section "Молниеносный индексатор"): special cases that reduce to a plain matrix
product, closed forms for the ReLU and the head weights, positive
homogeneity of the FP8 scales, causal masking and batch bookkeeping."""
import numpy as np
import pytest

import oracle
import synth


def _prefill(L, n_kv=None, pos0=0):
    b = synth.Batch.prefill(L, n_kv if n_kv is not None else L, pos0)
    return b.cu_q, b.cu_kv, b.pos0


def _causal_expect(M, pos0=0):
    """Expected scores given an unmasked full matrix M[t, s]: -inf past the
    query position."""
    T, N = M.shape
    out = M.astype(np.float32).copy()
    for t in range(T):
        out[t, min(pos0 + t + 1, N):] = -np.inf
    return out


def test_single_head_nonnegative_is_matmul():
    rng = np.random.default_rng(0)
    L, d = 40, 16
    q = np.abs(rng.standard_normal((L, 1, d))).astype(np.float32)
    k = np.abs(rng.standard_normal((L, d))).astype(np.float32)
    w = np.ones((L, 1), np.float32)
    got = oracle.indexer(*_prefill(L), q, None, w, k, None)
    ref = q[:, 0, :].astype(np.float64) @ k.T.astype(np.float64)
    assert np.array_equal(got, _causal_expect(ref))


def test_relu_closed_form_abs():
    # heads x and -x with unit weights: relu(a) + relu(-a) = |a|
    rng = np.random.default_rng(1)
    L, d = 33, 8
    x = rng.standard_normal((L, d)).astype(np.float32)
    q = np.stack([x, -x], axis=1)
    k = rng.standard_normal((L, d)).astype(np.float32)
    w = np.ones((L, 2), np.float32)
    got = oracle.indexer(*_prefill(L), q, None, w, k, None)
    ref = np.abs(x.astype(np.float64) @ k.T.astype(np.float64))
    assert np.array_equal(got, _causal_expect(ref))


def test_relu_drops_negative_products():
    # a single head with negated keys: every score is max(0, -x.k)
    rng = np.random.default_rng(2)
    L, d = 20, 8
    x = rng.standard_normal((L, 1, d)).astype(np.float32)
    k = rng.standard_normal((L, d)).astype(np.float32)
    w = np.full((L, 1), 0.5, np.float32)
    got = oracle.indexer(*_prefill(L), x, None, w, k, None)
    dots = x[:, 0].astype(np.float64) @ k.T.astype(np.float64)
    ref = 0.5 * np.maximum(dots, 0.0)
    assert np.array_equal(got, _causal_expect(ref))
    assert np.sum(_causal_expect(dots) < 0) > 0 and np.all(got[np.isfinite(got)] >= 0)


def test_head_weights_closed_form():
    # identical heads with weights a, b: (a + b) * relu(x.k), also for signed weights
    rng = np.random.default_rng(3)
    L, d = 25, 8
    x = rng.standard_normal((L, 1, d)).astype(np.float32)
    q = np.concatenate([x, x, x], axis=1)
    k = rng.standard_normal((L, d)).astype(np.float32)
    w = np.stack([np.full(L, 0.75), np.full(L, -2.0), np.full(L, 0.25)], axis=1).astype(np.float32)
    got = oracle.indexer(*_prefill(L), q, None, w, k, None)
    ref = -1.0 * np.maximum(x[:, 0].astype(np.float64) @ k.T.astype(np.float64), 0)
    assert np.array_equal(got, _causal_expect(ref))


def test_per_query_weights_select_rows():
    # weights differ per query: row t uses w[t], not w[s] (catches a transposed index)
    rng = np.random.default_rng(4)
    L, d = 16, 4
    q = np.abs(rng.standard_normal((L, 1, d))).astype(np.float32)
    k = np.abs(rng.standard_normal((L, d))).astype(np.float32)
    w = np.arange(1, L + 1, dtype=np.float32)[:, None]
    got = oracle.indexer(*_prefill(L), q, None, w, k, None)
    ref = np.arange(1, L + 1)[:, None] * (q[:, 0].astype(np.float64) @ k.T.astype(np.float64))
    assert np.array_equal(got, _causal_expect(ref))


def test_fp8_codes_equal_f32_values_when_exact():
    # power-of-two scales keep code*scale exact, so the FP8 path equals the f32 path
    rng = np.random.default_rng(5)
    L, HI, d = 30, 4, 32
    qc = rng.integers(0, 256, size=(L, HI, d), dtype=np.uint8)
    kc = rng.integers(0, 256, size=(L, d), dtype=np.uint8)
    qc[(qc & 0x7F) == 0x7F] = 0x38  # no NaN codes
    kc[(kc & 0x7F) == 0x7F] = 0x38
    qs = (2.0 ** rng.integers(-6, 4, size=(L, HI))).astype(np.float32)
    ks = (2.0 ** rng.integers(-6, 4, size=L)).astype(np.float32)
    w = rng.standard_normal((L, HI)).astype(np.float32)
    tab = oracle.e4m3_table()
    qf = (tab[qc] * qs[:, :, None]).astype(np.float32)
    kf = (tab[kc] * ks[:, None]).astype(np.float32)
    a = oracle.indexer(*_prefill(L), qc, qs, w, kc, ks)
    b = oracle.indexer(*_prefill(L), qf, None, w, kf, None)
    assert np.array_equal(a, b)


def test_scale_homogeneity():
    # I(alpha * s_k) = alpha * I and I(beta * s_q) = beta * I for alpha, beta > 0
    inp = synth.make_inputs(synth.Batch.prefill(48, 48, 0), seed=21, HI=8, DI=32, H=2, D=16, Dv=8)
    c = (inp.batch.cu_q, inp.batch.cu_kv, inp.batch.pos0)
    base = oracle.indexer(*c, inp.qi, inp.qi_scale, inp.w, inp.ki, inp.ki_scale).astype(np.float64)
    s1 = oracle.indexer(*c, inp.qi, inp.qi_scale, inp.w, inp.ki, inp.ki_scale * np.float32(4.0))
    s2 = oracle.indexer(*c, inp.qi, inp.qi_scale * np.float32(0.25), inp.w, inp.ki, inp.ki_scale)
    fin = np.isfinite(base)
    assert np.array_equal(s1[fin], (4.0 * base[fin]).astype(np.float32))
    assert np.array_equal(s2[fin], (0.25 * base[fin]).astype(np.float32))
    assert np.array_equal(np.isfinite(s1), fin)


def test_causal_mask_and_future_independence():
    inp = synth.make_inputs(synth.Batch.prefill(64, 64, 0), seed=22, HI=4, DI=32, H=2, D=16, Dv=8)
    c = (inp.batch.cu_q, inp.batch.cu_kv, inp.batch.pos0)
    s = oracle.indexer(*c, inp.qi, inp.qi_scale, inp.w, inp.ki, inp.ki_scale)
    t_idx, s_idx = np.meshgrid(np.arange(64), np.arange(64), indexing="ij")
    assert np.all(np.isneginf(s[s_idx > t_idx]))
    assert np.all(np.isfinite(s[s_idx <= t_idx]))
    # changing key rows 40.. leaves rows t < 40 unchanged
    k2 = inp.ki.copy()
    k2[40:] = 0x38
    s2 = oracle.indexer(*c, inp.qi, inp.qi_scale, inp.w, k2, inp.ki_scale)
    assert np.array_equal(s[:40], s2[:40])
    assert not np.array_equal(s[40:], s2[40:])


def test_abs_sum_equals_score_for_nonnegative_weights():
    inp = synth.make_inputs(synth.Batch.prefill(32, 32, 0), seed=23, HI=8, DI=32, H=2, D=16, Dv=8)
    c = (inp.batch.cu_q, inp.batch.cu_kv, inp.batch.pos0)
    w = np.abs(inp.w)
    s, A = oracle.indexer(*c, inp.qi, inp.qi_scale, w, inp.ki, inp.ki_scale, want_abs=True)
    fin = np.isfinite(s)
    assert np.array_equal(s[fin], A[fin].astype(np.float32))
    assert np.all(s[fin] >= 0)
    # with signed weights |I| <= A
    s, A = oracle.indexer(*c, inp.qi, inp.qi_scale, inp.w, inp.ki, inp.ki_scale, want_abs=True)
    assert np.all(np.abs(s[fin].astype(np.float64)) <= A[fin] * (1 + 1e-6) + 1e-30)
    assert np.any(s[fin] < 0)


@pytest.mark.parametrize("rows", [None, [0, 5, 7, 10]])
def test_ragged_batch_equals_separate_sequences(rows):
    # three sequences: chunked prefill, plain prefill, decode row
    b = synth.Batch.ragged([4, 6, 1], [10, 6, 9], [6, 0, 8])
    inp = synth.make_inputs(b, seed=24, HI=4, DI=32, H=2, D=16, Dv=8)
    allrows = np.arange(b.T) if rows is None else np.array(rows)
    got = oracle.indexer(b.cu_q, b.cu_kv, b.pos0, inp.qi, inp.qi_scale, inp.w, inp.ki,
                         inp.ki_scale, rows=rows, ld=10)
    for i, t in enumerate(allrows):
        bb = int(np.searchsorted(b.cu_q, t, side="right") - 1)
        q0, q1 = int(b.cu_q[bb]), int(b.cu_q[bb + 1])
        k0, k1 = int(b.cu_kv[bb]), int(b.cu_kv[bb + 1])
        single = oracle.indexer([0, q1 - q0], [0, k1 - k0], [int(b.pos0[bb])], inp.qi[q0:q1],
                                inp.qi_scale[q0:q1], inp.w[q0:q1], inp.ki[k0:k1], inp.ki_scale[k0:k1])
        n = k1 - k0
        assert np.array_equal(got[i, :n], single[t - q0, :n], equal_nan=True)
        assert np.all(np.isnan(got[i, n:]))  # beyond the context: untouched


def test_tiny_config_brute_force_loops():
    # pure-Python loops on a small slice of the tiny configuration
    inp = synth.tiny_prefill()
    b = inp.batch
    s = oracle.indexer(b.cu_q, b.cu_kv, b.pos0, inp.qi, None, inp.w, inp.ki, None, rows=[0, 17, 255])
    for i, t in enumerate([0, 17, 255]):
        for sk in [0, t // 2, t]:
            tot = 0.0
            for j in range(inp.HI):
                dot = sum(float(inp.qi[t, j, d]) * float(inp.ki[sk, d]) for d in range(inp.DI))
                tot += float(inp.w[t, j]) * (dot if dot > 0 else 0.0)
            assert abs(s[i, sk] - tot) <= 1e-6 * max(1.0, abs(tot))
