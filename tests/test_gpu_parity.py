"""GPU parity of the HIP path against the CPU oracle, called through the C ABI.

Small cases (the oracle computes every row) span several row blocks, key tiles
and ragged tails; edge cases cover single-key rows, rows of exactly k and k+1
keys, exact ties, empty selections, long rows that need chunked selection, and
split-KV attention.  Tolerances are documented in tests/gpu_util.py.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import (DevInputs, bf16_to_f32, check_attention, check_idx_sets, check_scores,
                      dev, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsa():
    import sparse_attention_16_amd as m  # fails loudly when libdsa.so is missing
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def _ref_scores(inp, rows=None, ld=None):
    b = inp.batch
    return oracle.indexer(b.cu_q, b.cu_kv, b.pos0, inp.qi, inp.qi_scale, inp.w, inp.ki,
                          inp.ki_scale, rows=rows, ld=ld, want_abs=True)


def _nvis(inp, rows=None):
    b = inp.batch
    _, _, ctx, _, nvis = oracle.visible(b.cu_q, b.cu_kv, b.pos0)
    if rows is not None:
        return nvis[rows], ctx[rows]
    return nvis, ctx


# ------------------------------------------------------------------ indexer

INDEXER_CASES = {
    "prefill_300": lambda: synth.make_inputs(synth.Batch.prefill(300, 300, 0), seed=101, k=64),
    "chunked_40_at_960": lambda: synth.make_inputs(synth.Batch.prefill(40, 1000, 960), seed=102, k=64),
    "ragged_3seq": lambda: synth.make_inputs(synth.Batch.ragged([20, 1, 37], [50, 9, 300], [30, 8, 263]),
                                             seed=103, k=64),
    "decode_edges": lambda: synth.make_inputs(synth.Batch.decode([1, 17, 300, 2048, 2049, 5000]),
                                              seed=104, k=64, per_seq=True),
}


@pytest.mark.parametrize("case", sorted(INDEXER_CASES))
def test_indexer_scores(dsa, case):
    say(f"[indexer] {case}")
    inp = INDEXER_CASES[case]()
    d = DevInputs(inp, dsa)
    ld = ((inp.batch.max_kv + 15) // 16) * 16 + 16
    scores = torch.full((inp.batch.T, ld), float("nan"), device="cuda")
    dsa.indexer_scores(d.batch, d.qi, d.qs, d.w, d.ki, d.ks, scores)
    torch.cuda.synchronize()
    g = scores.cpu().numpy()
    ref, A = _ref_scores(inp, ld=ld)
    nvis, ctx = _nvis(inp)
    worst = check_scores(g, ref, A, nvis, case)
    for r in range(inp.batch.T):
        n, c = int(nvis[r]), int(ctx[r])
        assert np.all(np.isneginf(g[r, n:c])), f"row {r}: masked columns must be -inf"
        assert np.all(np.isnan(g[r, c:])), f"row {r}: columns past the context must be untouched"
    say(f"  worst relative score error {worst:.3g}")


def test_indexer_duplicate_keys_bitwise(dsa):
    # identical key rows must give bit-identical GPU scores (exact ties survive)
    inp = synth.make_inputs(synth.Batch.prefill(64, 600, 536), seed=105, k=64)
    for a, b in [(3, 400), (77, 599), (250, 251)]:
        inp.ki[b] = inp.ki[a]
        inp.ki_scale[b] = inp.ki_scale[a]
    d = DevInputs(inp, dsa)
    scores = torch.empty((64, 600), device="cuda")
    dsa.indexer_scores(d.batch, d.qi, d.qs, d.w, d.ki, d.ks, scores)
    g = scores.cpu().numpy()
    for a, b in [(3, 400), (77, 599), (250, 251)]:
        vis = np.arange(64) + 536 >= b
        assert np.array_equal(g[vis, a], g[vis, b])


# -------------------------------------------------------------------- top-k

def _topk_case(name):
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    if name == "prefill_2100_k2048":
        b, k = synth.Batch.prefill(2100, 2100, 0), 2048
    elif name == "prefill_300_k64":
        b, k = synth.Batch.prefill(300, 300, 0), 64
    elif name == "long_rows_k2048":
        b, k = synth.Batch.decode([32768, 32769, 40000, 70001, 131072, 2049]), 2048
    elif name == "k1_and_k7":
        b, k = synth.Batch.prefill(50, 50, 0), 7
    else:
        raise KeyError(name)
    _, _, ctx, _, nvis = oracle.visible(b.cu_q, b.cu_kv, b.pos0)
    ld = int(b.max_kv)
    s = rng.standard_normal((b.T, ld)).astype(np.float32)
    # exact ties: a few repeated values per row, signed zeros, and -inf entries
    s[:, ::17] = np.float32(0.75)
    s[:, 5::23] = np.float32(-0.0)
    s[:, 7::29] = np.float32(0.0)
    s[:, 11::31] = -np.inf
    for r in range(b.T):
        s[r, nvis[r]:] = -np.inf
    return b, k, s


@pytest.mark.parametrize("name", ["prefill_300_k64", "prefill_2100_k2048", "long_rows_k2048",
                                  "k1_and_k7"])
def test_topk_bit_exact(dsa, name):
    say(f"[topk] {name}")
    b, k, s = _topk_case(name)
    ks = [k] if name != "k1_and_k7" else [1, 7]
    for kk in ks:
        ref = oracle.topk(b.cu_q, b.cu_kv, b.pos0, s, kk)
        batch = dsa.Batch.from_host(b.cu_q, b.cu_kv, b.pos0)
        idx = torch.full((b.T, kk), -7, dtype=torch.int32, device="cuda")
        dsa.topk(batch, dev(s), kk, idx)
        g = idx.cpu().numpy()
        assert np.array_equal(g, ref), f"{name} k={kk}: {np.sum(np.any(g != ref, axis=1))} rows differ"


def test_topk_all_equal_rows(dsa):
    b = synth.Batch.decode([5000, 40000])
    s = np.zeros((2, 40000), np.float32)
    s[0, 5000:] = -np.inf
    s[1, ::2] = -0.0
    batch = dsa.Batch.from_host(b.cu_q, b.cu_kv, b.pos0)
    idx = torch.empty((2, 2048), dtype=torch.int32, device="cuda")
    dsa.topk(batch, dev(s), 2048, idx)
    g = idx.cpu().numpy()
    assert np.array_equal(g[0], np.arange(2048)) and np.array_equal(g[1], np.arange(2048))


def _finite_topk_case(name):
    """Finite scores (the value-binned path; -inf among the visible columns
    sends a row to the radix path instead)."""
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    k = 2048
    if name == "finite_small_k":
        b, k = synth.Batch.prefill(300, 300, 0), 7   # the k-th key sits in the top bin
    elif name == "finite_prefill_2100":
        b = synth.Batch.prefill(2100, 2100, 0)
    elif name == "finite_long_rows":
        b = synth.Batch.decode([32768, 32769, 40000, 70001, 131072, 2049])
    elif name == "binary_scores":
        b = synth.Batch.decode([32768, 40000, 9000, 70001])
    else:
        b = synth.Batch.decode([3000, 17000, 30721, 32768, 50000])
    _, _, ctx, _, nvis = oracle.visible(b.cu_q, b.cu_kv, b.pos0)
    s = rng.standard_normal((b.T, int(b.max_kv))).astype(np.float32)
    if name.startswith("finite"):
        s[:, ::17] = np.float32(0.75)
        s[:, 5::23] = np.float32(-0.0)
        s[:, 7::29] = np.float32(0.0)
    elif name.startswith("kappa_ties"):
        # 2t keys around rank k share the k-th value: the tie at the boundary
        # is broken by column, across the whole row (and across chunks)
        t = int(name.rsplit("_", 1)[1]) // 2
        for r in range(b.T):
            n = int(nvis[r])
            order = np.argsort(-s[r, :n], kind="stable")
            s[r, order[k - 1 - t:k - 1 + t]] = s[r, order[k - 1]]
    elif name == "binary_scores":
        # 30% of the scores 1, the rest 0: the k-th largest is tied with about
        # 10k keys of a 32768-column chunk, more candidates than the sampled
        # threshold path takes, so the chunk goes through the radix fallback
        s = (rng.random(s.shape) < 0.3).astype(np.float32)
    elif name == "sub_ulp_bins":
        # a range of a few float ulps: value bins narrower than the spacing of
        # the scores, most scores tied
        s = (np.float32(1000.0) + np.float32(2e-4) * s).astype(np.float32)
    else:
        raise KeyError(name)
    for r in range(b.T):
        s[r, nvis[r]:] = -np.inf
    return b, k, s


@pytest.mark.parametrize("name", ["finite_small_k", "finite_prefill_2100", "finite_long_rows", "kappa_ties_300",
                                  "kappa_ties_900", "sub_ulp_bins", "binary_scores"])
def test_topk_bit_exact_finite_scores(dsa, name):
    say(f"[topk] {name}")
    b, k, s = _finite_topk_case(name)
    for kk in ([1, k] if name == "finite_small_k" else [k]):
        ref = oracle.topk(b.cu_q, b.cu_kv, b.pos0, s, kk)
        batch = dsa.Batch.from_host(b.cu_q, b.cu_kv, b.pos0)
        idx = torch.full((b.T, kk), -7, dtype=torch.int32, device="cuda")
        dsa.topk(batch, dev(s), kk, idx)
        g = idx.cpu().numpy()
        assert np.array_equal(g, ref), f"{name} k={kk}: {np.sum(np.any(g != ref, axis=1))} rows differ"


# ---------------------------------------------------------------- attention

def _attn_case(name):
    if name == "prefill_300_k64":
        inp = synth.make_inputs(synth.Batch.prefill(300, 300, 0), seed=111, k=64)
    elif name == "decode_6_k2048":
        inp = synth.make_inputs(synth.Batch.decode([1, 100, 2048, 2049, 9000, 40000]), seed=112,
                                k=2048, per_seq=True)
    elif name == "prefill_700_k256":
        inp = synth.make_inputs(synth.Batch.prefill(700, 700, 0), seed=113, k=256)
    else:
        raise KeyError(name)
    return inp


@pytest.mark.parametrize("name", ["prefill_300_k64", "decode_6_k2048", "prefill_700_k256"])
def test_sparse_mla_on_oracle_idx(dsa, name):
    say(f"[sparse_mla] {name}")
    inp = _attn_case(name)
    b = inp.batch
    ref_s, A = _ref_scores(inp)
    idx = oracle.topk(b.cu_q, b.cu_kv, b.pos0, ref_s, inp.k)
    o_ref, lse_ref = oracle.sparse_attn(b.cu_q, b.cu_kv, b.pos0, inp.q, inp.kv, idx, inp.Dv, inp.scale)
    d = DevInputs(inp, dsa)
    out = torch.empty((b.T, inp.H, inp.Dv), dtype=torch.int16, device="cuda")
    lse = torch.empty((b.T, inp.H), dtype=torch.float32, device="cuda")
    dsa.sparse_mla_fwd(d.batch, d.q, d.kv, dev(idx), inp.scale, out, lse)
    torch.cuda.synchronize()
    dl, rel = check_attention(bf16_to_f32(out), lse.cpu().numpy(), o_ref, lse_ref, name)
    say(f"  max |dlse| {dl:.3g}, max row ||do||/||o|| {rel:.3g}")


def test_sparse_mla_holes_and_empty_rows(dsa):
    # -1 anywhere, out-of-range entries skipped, an all -1 row, duplicates
    inp = synth.make_inputs(synth.Batch.prefill(40, 3000, 2960), seed=114, k=100)
    b = inp.batch
    rng = np.random.default_rng(5)
    idx = rng.integers(0, 2961, size=(40, 100)).astype(np.int32)
    idx[rng.random((40, 100)) < 0.2] = -1
    idx[3] = -1
    idx[7, :10] = 5  # duplicates count as many times as listed
    ref_idx = idx.copy()
    o_ref, lse_ref = oracle.sparse_attn(b.cu_q, b.cu_kv, b.pos0, inp.q, inp.kv, ref_idx, inp.Dv,
                                        inp.scale)
    bad = idx.copy()
    bad[9, 50] = 3000   # >= ctx: skipped by the GPU path
    bad[9, 51] = -5
    ref9 = ref_idx[9].copy()
    ref9[50] = -1
    ref9[51] = -1
    o9, l9 = oracle.sparse_attn(b.cu_q, b.cu_kv, b.pos0, inp.q, inp.kv, ref9[None], inp.Dv, inp.scale,
                                rows=[9])
    o_ref[9], lse_ref[9] = o9[0], l9[0]
    d = DevInputs(inp, dsa)
    out = torch.empty((40, 128, 512), dtype=torch.int16, device="cuda")
    lse = torch.empty((40, 128), device="cuda")
    dsa.sparse_mla_fwd(d.batch, d.q, d.kv, dev(bad), inp.scale, out, lse)
    check_attention(bf16_to_f32(out), lse.cpu().numpy(), o_ref, lse_ref, "holes")
    assert np.all(np.isneginf(lse.cpu().numpy()[3]))


@pytest.mark.parametrize("T,amp", [(512, 0x43C8), (512, 0x4416), (40, 0x4416)])
def test_sparse_mla_reference_restart(dsa, T, amp):
    """A selected key whose logit exceeds the first block's maximum by more
    than the kernel's headroom (64 in log2 units) must trigger the exact
    second pass.  Every query head gets a strong component along dim 0 and one
    cache row a large dim-0 value: its logit is about 50 (natural units) while
    the others stay near N(0, 1) (amp = bf16 400: about 62..78 log2 units
    above the first block, around the headroom; bf16 600: far above).  The
    row's position in the selected set
    varies: first block (no restart), middle, last.  T=512 runs one split per
    row; T=40 splits the selected set (the merge sees very different lse)."""
    say(f"[sparse_mla restart] T={T} amp={amp:#x}")
    N = 3000
    inp = synth.make_inputs(synth.Batch.prefill(T, N, N - T), seed=115, k=256)
    b = inp.batch
    big = 1500
    q = inp.q.copy()
    q[:, :, 0] = np.uint16(0x4040)           # 3.0 in bf16
    kv = inp.kv.copy()
    kv[big, 0] = np.uint16(amp)
    rng = np.random.default_rng(9)
    idx = np.empty((T, 256), np.int32)
    for t in range(T):
        cand = rng.choice(np.setdiff1d(np.arange(N - T + t + 1), [big]), size=255, replace=False)
        row = np.sort(np.append(cand, big)).astype(np.int32)
        pos = [3, 130, 250][t % 3]           # where the big row lands in the selected set
        row = np.delete(row, np.searchsorted(row, big))
        idx[t] = np.insert(row, pos, big)
    o_ref, lse_ref = oracle.sparse_attn(b.cu_q, b.cu_kv, b.pos0, q, kv, idx, inp.Dv, inp.scale)
    assert float(np.max(lse_ref)) > 40.0      # the jump is really there
    batch = dsa.Batch.from_host(b.cu_q, b.cu_kv, b.pos0)
    out = torch.empty((T, 128, 512), dtype=torch.int16, device="cuda")
    lse = torch.empty((T, 128), device="cuda")
    dsa.sparse_mla_fwd(batch, dev(q), dev(kv), dev(idx), inp.scale, out, lse)
    torch.cuda.synchronize()
    dl, rel = check_attention(bf16_to_f32(out), lse.cpu().numpy(), o_ref, lse_ref, f"restart T={T} amp={amp:#x}")
    say(f"  max |dlse| {dl:.3g}, max row ||do||/||o|| {rel:.3g}")


# ------------------------------------------------------------ fused entries

def _check_fused(dsa, inp, entry, rows=None, what=""):
    b = inp.batch
    d = DevInputs(inp, dsa)
    args = dsa.fwd_args(d.batch, d.qi, d.qs, d.w, d.ki, d.ks, d.q, d.kv, inp.k, inp.scale)
    out = torch.empty((b.T, inp.H, inp.Dv), dtype=torch.int16, device="cuda")
    lse = torch.empty((b.T, inp.H), device="cuda")
    idx = torch.empty((b.T, inp.k), dtype=torch.int32, device="cuda")
    fn = dsa.prefill_fwd if entry == "prefill" else dsa.decode_fwd
    fn(args, d.batch, out, lse, idx)
    torch.cuda.synchronize()
    say(f"  {what}: GPU done")
    rsel = np.arange(b.T) if rows is None else np.asarray(rows)
    g_idx = idx.cpu().numpy()[rsel]
    g_out = bf16_to_f32(out[torch.as_tensor(rsel, device="cuda")])
    g_lse = lse.cpu().numpy()[rsel]
    ref_s, A = _ref_scores(inp, rows=None if rows is None else rsel)
    ref_idx = oracle.topk(b.cu_q, b.cu_kv, b.pos0, ref_s, inp.k, rows=None if rows is None else rsel)
    nvis, _ = _nvis(inp, rsel)
    differ = check_idx_sets(g_idx, ref_idx, ref_s, A, nvis, inp.k, what)
    say(f"  {what}: {len(rsel)} rows, {len(differ)} differ only at near-ties")
    assert len(differ) <= max(2, len(rsel) // 20)
    same = np.setdiff1d(np.arange(len(rsel)), differ)
    o_ref, lse_ref = oracle.sparse_attn(b.cu_q, b.cu_kv, b.pos0, inp.q, inp.kv, ref_idx[same],
                                        inp.Dv, inp.scale, rows=rsel[same])
    dl, rel = check_attention(g_out[same], g_lse[same], o_ref, lse_ref, what)
    say(f"  {what}: max |dlse| {dl:.3g}, max row ||do||/||o|| {rel:.3g}")
    if differ:
        # rows whose set differs at near-ties: the same kernel on the oracle's set
        fix = idx.clone()
        fix[torch.as_tensor(rsel[differ], device="cuda")] = dev(ref_idx[differ])
        out2 = torch.empty_like(out)
        lse2 = torch.empty_like(lse)
        dsa.sparse_mla_fwd(d.batch, d.q, d.kv, fix, inp.scale, out2, lse2)
        o_r, l_r = oracle.sparse_attn(b.cu_q, b.cu_kv, b.pos0, inp.q, inp.kv, ref_idx[differ],
                                      inp.Dv, inp.scale, rows=rsel[differ])
        sel = torch.as_tensor(rsel[differ], device="cuda")
        check_attention(bf16_to_f32(out2[sel]), lse2[sel].cpu().numpy(), o_r, l_r, what + " (oracle set)")


def test_prefill_fwd_small(dsa):
    say("[prefill_fwd] L=600 k=128")
    inp = synth.make_inputs(synth.Batch.prefill(600, 600, 0), seed=121, k=128)
    _check_fused(dsa, inp, "prefill", what="prefill L=600 k=128")


def test_prefill_fwd_ragged_batch(dsa):
    say("[prefill_fwd] ragged 3 sequences k=64")
    inp = synth.make_inputs(synth.Batch.ragged([70, 1, 33], [200, 90, 33], [130, 89, 0]),
                            seed=122, k=64)
    _check_fused(dsa, inp, "prefill", what="ragged k=64")


def test_decode_fwd_mixed(dsa):
    say("[decode_fwd] B=6 mixed contexts k=2048")
    inp = synth.make_inputs(synth.Batch.decode([1, 2048, 2049, 20000, 40000, 70000]), seed=123,
                            k=2048, per_seq=True)
    _check_fused(dsa, inp, "decode", what="decode mixed")


# ------------------------------------------------- indexer key-chunk widths

def _indexer_width_case(width):
    """1024 sequences of 16 query rows: one sequence long enough that the
    prefill indexer takes `width` keys per workgroup (at least 8 workgroups per
    compute unit over 1024 row blocks x its key chunks), the others short.  The
    long sequence's queries sit mid-context, so its rows have a causally masked
    stretch that crosses the chunk boundary, then the columns past its context."""
    B = 1024
    rng = np.random.default_rng(width)
    long_ctx = {4096: 6000, 8192: 12000}[width]
    n_kv = rng.integers(20, 200, size=B)
    n_kv[0] = long_ctx
    pos0 = np.maximum(n_kv - 16 - rng.integers(0, 8, size=B), 0)
    pos0[0] = long_ctx // 2 - 100
    return synth.Batch.ragged(np.full(B, 16), n_kv, pos0)


@pytest.mark.parametrize("width", [4096, 8192])
def test_indexer_chunk_widths(dsa, width):
    """The prefill indexer's 4096- and 8192-key workgroup widths (chosen by
    the row blocks x key chunks of the batch): sampled rows against the oracle,
    -inf over the masked columns [nvis, ctx), columns past ctx untouched."""
    say(f"[indexer] chunk width {width}")
    b = _indexer_width_case(width)
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    rowblocks = ((b.max_q + 15) // 16) * b.B
    chosen = next((c for c in (8192, 4096) if rowblocks * -(-b.max_kv // c) >= 8 * ncu), 2048)
    say(f"  {ncu} compute units: {chosen} keys per workgroup expected")
    if ncu == 256:
        assert chosen == width
    wl = synth.Workload(b, seed=131 + width, k=64)
    qi, qs = wl.qi_rows(0, b.T)
    ki, ks = wl.ki_rows(0, b.N)
    w = wl.w_rows(0, b.T)
    batch = dsa.Batch.from_host(b.cu_q, b.cu_kv, b.pos0)
    ld = ((b.max_kv + 63) // 64) * 64 + 64
    scores = torch.full((b.T, ld), float("nan"), device="cuda")
    dsa.indexer_scores(batch, dev(qi), dev(qs), dev(w), dev(ki), dev(ks), scores)
    torch.cuda.synchronize()
    rows = np.concatenate([np.arange(16), np.sort(np.random.default_rng(7).choice(
        np.arange(16, b.T), 200, replace=False))])
    g = scores[torch.as_tensor(rows, device="cuda")].cpu().numpy()
    ref, A = oracle.indexer(b.cu_q, b.cu_kv, b.pos0, qi, qs, w, ki, ks, rows=rows, ld=ld, want_abs=True)
    _, _, ctx, _, nvis = oracle.visible(b.cu_q, b.cu_kv, b.pos0)
    worst = check_scores(g, ref, A, nvis[rows], f"width {width}")
    for i, r in enumerate(rows):
        n, c = int(nvis[r]), int(ctx[r])
        assert np.all(np.isneginf(g[i, n:c])), f"row {r}: masked columns must be -inf"
        assert np.all(np.isnan(g[i, c:])), f"row {r}: columns past the context must be untouched"
    say(f"  worst relative score error {worst:.3g}")


# ------------------------------ fused entries == the three separate steps

FUSED_LONG = {
    "decode_long_rows": lambda: synth.make_inputs(
        synth.Batch.decode([32769, 40000, 70001, 131072, 2049, 5000, 100000, 65536]), seed=141, k=2048,
        per_seq=True),
    "chunked_48_at_65488": lambda: synth.make_inputs(synth.Batch.prefill(48, 65536, 65488), seed=142, k=2048),
}


@pytest.mark.parametrize("name", sorted(FUSED_LONG))
def test_fused_idx_equals_three_steps(dsa, name):
    """The fused entries' selection equals dsa_indexer_scores + dsa_topk on the
    same inputs bit for bit, on rows longer than one 32768-column select chunk
    (the scores are the same fp32 values, so the exact top-k is the same set)."""
    say(f"[fused == three steps] {name}")
    inp = FUSED_LONG[name]()
    b = inp.batch
    d = DevInputs(inp, dsa)
    entry = "decode" if name.startswith("decode") else "prefill"
    args = dsa.fwd_args(d.batch, d.qi, d.qs, d.w, d.ki, d.ks, d.q, d.kv, inp.k, inp.scale)
    out = torch.empty((b.T, inp.H, inp.Dv), dtype=torch.int16, device="cuda")
    lse = torch.empty((b.T, inp.H), device="cuda")
    idx = torch.full((b.T, inp.k), -7, dtype=torch.int32, device="cuda")
    (dsa.decode_fwd if entry == "decode" else dsa.prefill_fwd)(args, d.batch, out, lse, idx)
    ld = ((b.max_kv + 63) // 64) * 64
    scores = torch.empty((b.T, ld), device="cuda")
    dsa.indexer_scores(d.batch, d.qi, d.qs, d.w, d.ki, d.ks, scores)
    idx3 = torch.full((b.T, inp.k), -9, dtype=torch.int32, device="cuda")
    dsa.topk(d.batch, scores, inp.k, idx3)
    torch.cuda.synchronize()
    g, g3 = idx.cpu().numpy(), idx3.cpu().numpy()
    assert np.array_equal(g, g3), f"{name}: {np.sum(np.any(g != g3, axis=1))} rows differ"
    _, _, ctx, _, nvis = oracle.visible(b.cu_q, b.cu_kv, b.pos0)
    assert np.any(nvis > 32768)
    say(f"  {b.T} rows, longest {int(nvis.max())} keys: identical")
