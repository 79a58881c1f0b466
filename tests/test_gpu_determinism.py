"""Run-twice determinism of every GPU entry point: two calls on the same
inputs give outputs identical bit for bit, with the workspace filled with a
different byte pattern before each call (so no result may depend on what the
workspace held, and nothing may depend on the order in which workgroups run
or atomics land).  The outputs are filled with the same pattern before both
calls, so parts an entry leaves untouched by contract compare equal.

Covered: the fused prefill and decode entries (rows past one select chunk,
rows with and without a sampled threshold, the wave and workgroup selects),
dsa_indexer_topk, dsa_indexer_scores, dsa_topk, dsa_sparse_mla_fwd,
dsa_dense_mla_fwd, dsa_indexer_kl_fwd, dsa_sparse_mla_bwd (whose dkv sums
run in a fixed order whatever order its slot counters are claimed in),
dsa_quantize_queries and dsa_append_cache.
"""
import numpy as np
import pytest
import torch

import synth
from gpu_util import DevInputs, dev, say

pytestmark = pytest.mark.gpu

WS_FILLS = (0xA5, 0x5A)
OUT_FILL = 0x3C


@pytest.fixture(scope="module")
def dsa():
    import sparse_attention_16_amd as m  # fails loudly when libdsa.so is missing
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def _bytes(t):
    return t.contiguous().view(torch.uint8)


def _twice(call, outs, ws_bytes, what):
    """call(ws) twice; outs (tensors it writes) must come out identical."""
    ws = torch.empty(max(int(ws_bytes), 1), dtype=torch.uint8, device="cuda") if ws_bytes else None
    runs = []
    for fill in WS_FILLS:
        for o in outs:
            _bytes(o).fill_(OUT_FILL)
        if ws is not None:
            ws.fill_(fill)
        call(ws)
        torch.cuda.synchronize()
        runs.append([o.clone() for o in outs])
    for i, (a, b) in enumerate(zip(*runs)):
        same = torch.equal(_bytes(a), _bytes(b))
        assert same, f"{what}: output {i} differs between two calls"
    say(f"  {what}: {len(outs)} outputs identical over two calls")


PREFILL = {
    # 3000 causal rows: rows up to 2048 take every key, up to 4096 no threshold
    "prefill_3000": lambda: synth.make_inputs(synth.Batch.prefill(3000, 3000, 0), seed=181, k=2048),
    # 1536 rows at the end of a 40000-key context: thresholds, rows past one
    # 32768-column select chunk, more rows than the workgroup select takes
    "chunked_1536_at_40000": lambda: synth.make_inputs(synth.Batch.prefill(1536, 40000, 38464), seed=182,
                                                       k=2048),
}


def _fused(dsa, inp, entry):
    b = inp.batch
    d = DevInputs(inp, dsa)
    args = dsa.fwd_args(d.batch, d.qi, d.qs, d.w, d.ki, d.ks, d.q, d.kv, inp.k, inp.scale)
    out = torch.empty((b.T, inp.H, inp.Dv), dtype=torch.int16, device="cuda")
    lse = torch.empty((b.T, inp.H), device="cuda")
    idx = torch.empty((b.T, inp.k), dtype=torch.int32, device="cuda")
    ws_entry = dsa.WS_PREFILL if entry == "prefill" else dsa.WS_DECODE
    fn = dsa.prefill_fwd if entry == "prefill" else dsa.decode_fwd
    need = dsa.workspace_size(ws_entry, d.batch, inp.k)
    _twice(lambda ws: fn(args, d.batch, out, lse, idx, ws=ws), [out, lse, idx], need, f"{entry}_fwd")
    return d, out, lse, idx


@pytest.mark.parametrize("name", sorted(PREFILL))
def test_prefill_fwd_twice(dsa, name):
    say(f"[determinism] prefill_fwd {name}")
    _fused(dsa, PREFILL[name](), "prefill")


def test_decode_fwd_twice(dsa):
    say("[determinism] decode_fwd, 8 sequences of 1 to 100000 keys")
    inp = synth.make_inputs(synth.Batch.decode([32769, 70001, 2049, 5000, 100000, 1, 2048, 40000]), seed=183,
                            k=2048, per_seq=True)
    _fused(dsa, inp, "decode")


@pytest.mark.parametrize("name", sorted(PREFILL))
def test_separate_steps_twice(dsa, name):
    """indexer_topk, indexer_scores, topk, sparse_mla_fwd, indexer_kl_fwd and
    sparse_mla_bwd, each called twice on the same inputs."""
    say(f"[determinism] separate entries {name}")
    inp = PREFILL[name]()
    b = inp.batch
    d = DevInputs(inp, dsa)
    k = inp.k

    idx_f = torch.empty((b.T, k), dtype=torch.int32, device="cuda")
    need = dsa.workspace_size(dsa.WS_INDEXER_TOPK, d.batch, k)
    _twice(lambda ws: dsa.indexer_topk(d.batch, d.qi, d.qs, d.w, d.ki, d.ks, k, idx_f, ws=ws), [idx_f], need,
           "indexer_topk")

    ld = ((b.max_kv + 63) // 64) * 64
    scores = torch.empty((b.T, ld), device="cuda")
    _twice(lambda ws: dsa.indexer_scores(d.batch, d.qi, d.qs, d.w, d.ki, d.ks, scores), [scores], 0,
           "indexer_scores")

    idx = torch.empty((b.T, k), dtype=torch.int32, device="cuda")
    need = dsa.workspace_size(dsa.WS_TOPK, d.batch, k)
    _twice(lambda ws: dsa.topk(d.batch, scores, k, idx, ws=ws), [idx], need, "topk")
    assert torch.equal(idx, idx_f), "indexer_topk and indexer_scores + topk select different keys"

    out = torch.empty((b.T, inp.H, inp.Dv), dtype=torch.int16, device="cuda")
    lse = torch.empty((b.T, inp.H), device="cuda")
    need = dsa.workspace_size(dsa.WS_SPARSE_MLA, d.batch, k)
    _twice(lambda ws: dsa.sparse_mla_fwd(d.batch, d.q, d.kv, idx, inp.scale, out, lse, ws=ws), [out, lse], need,
           "sparse_mla_fwd")

    # KL over the selected keys: scores past a context are never read, zero them
    sc = torch.nan_to_num(scores, nan=0.0)
    kl = torch.empty(b.T, device="cuda")
    p = torch.empty((b.T, k), device="cuda")
    need = dsa.workspace_size(dsa.WS_INDEXER_KL, d.batch, k)
    _twice(lambda ws: dsa.indexer_kl_fwd(d.batch, d.q, d.kv, lse, inp.scale, sc, kl, idx=idx, p_out=p, ws=ws),
           [kl, p], need, "indexer_kl_fwd")

    g = torch.Generator(device="cpu").manual_seed(184)
    dout = torch.randn((b.T, inp.H, inp.Dv), generator=g).to(torch.bfloat16).view(torch.int16).cuda()
    dq = torch.empty((b.T, inp.H, inp.D), device="cuda")
    dkv = torch.empty((b.N, inp.D), device="cuda")
    need = dsa.workspace_size(dsa.WS_SPARSE_MLA_BWD, d.batch, k)
    _twice(lambda ws: dsa.sparse_mla_bwd(d.batch, d.q, d.kv, idx, inp.scale, out, lse, dout, dq, dkv, ws=ws),
           [dq, dkv], need, "sparse_mla_bwd")


def test_dense_mla_twice(dsa):
    say("[determinism] dense_mla_fwd L=1500")
    inp = synth.make_inputs(synth.Batch.prefill(1500, 1500, 0), seed=185, k=2048)
    b = inp.batch
    d = DevInputs(inp, dsa)
    out = torch.empty((b.T, inp.H, inp.Dv), dtype=torch.int16, device="cuda")
    lse = torch.empty((b.T, inp.H), device="cuda")
    need = dsa.workspace_size(dsa.WS_DENSE_MLA, d.batch, inp.k)
    _twice(lambda ws: dsa.dense_mla_fwd(d.batch, d.q, d.kv, inp.scale, out, lse, ws=ws), [out, lse], need,
           "dense_mla_fwd")


def test_quantize_and_append_twice(dsa):
    say("[determinism] quantize_queries, append_cache")
    rng = np.random.default_rng(186)
    q = dev(rng.standard_normal((700, 64, 128)).astype(np.float32))
    q8 = torch.empty((700, 64, 128), dtype=torch.uint8, device="cuda")
    qs = torch.empty((700, 64), device="cuda")
    _twice(lambda ws: dsa.quantize_queries(q, q8, qs), [q8, qs], 0, "quantize_queries")

    N, R = 5000, 333
    k_new = dev(rng.standard_normal((R, 128)).astype(np.float32))
    kv_new = torch.from_numpy(rng.standard_normal((R, 576)).astype(np.float32)).to(torch.bfloat16) \
        .view(torch.int16).cuda()
    dst = torch.from_numpy(rng.choice(N, R, replace=False).astype(np.int64)).cuda()
    k8 = torch.empty((N, 128), dtype=torch.uint8, device="cuda")
    ks = torch.empty(N, device="cuda")
    kv = torch.empty((N, 576), dtype=torch.int16, device="cuda")
    _twice(lambda ws: dsa.append_cache(k_new, kv_new, dst, k8, ks, kv), [k8, ks, kv], 0, "append_cache")
