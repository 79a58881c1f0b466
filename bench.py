"""DSA hot-path benchmark on one MI355X: indexer + top-2048 + sparse MQA MLA.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload headline]

A step is one call of the fused C-ABI entry (dsa_prefill_fwd, or dsa_decode_fwd
for the decode workload) over one batch of synthetic inputs already resident
in HBM.  Prints one JSON line: tokens/s over the K timed steps, every kernel
of the step timed with HIP events recorded around its own launches on the
stream it runs on (dsa_fwd_profile; mean and median over >= 20 calls), the
roofline of the kernel with the largest time, the step's event median with
and without an Infinity Cache flush, and the CPU oracle timed on a bounded
sample of the same workload on this host's cores.

The default workload, headline, is the metric's pair: `value` is the 32K
prefill (one sequence of 32768 tokens), and the line nests the same figures
for the decode batch (64 sequences, one new token each) under "decode_64k".

Workloads (synthetic, seeded; the shapes and distributions of the DSA
configurations): prefill_32k, prefill_4k, decode_64k (64 sequences,
contexts uniform in 16384..131072, one new token each), chunked_128k (4096 new
tokens at the end of a 131072-entry context), short_prefill_2k (the
short-sequence mode), and the neighbours of the path: quant_append_32k,
indexer_kl_32k, sparse_bwd_32k.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "DSA tokens/s (indexer+top-2048+sparse MLA), 32K prefill & 64K-ctx decode"

# MI355X published peaks
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP8_TFLOPS = 5000.0
PEAK_HBM_GBS = 8000.0

HI, DI, H, D, DV = 64, 128, 128, 576, 512
SEED_QUANT = 0xD5A6        # seed of the quantise + append inputs
SEED_SHORT = 0xD5A7        # seed of the short-prompt (2048-token) prefill

# HBM traffic of the dominant kernel per launch, from rocprofv3 --pmc runs
# (FETCH_SIZE, then WRITE_SIZE, in KiB per dispatch, one run each).  The raw
# counters are scaled by what the same counters read for a plain 1 GiB
# device-to-device copy (bench.py --copy-calibration): FETCH_SIZE reads
# 524300 KiB for the 1 GiB read (x2.0), WRITE_SIZE 1048576 KiB (x1.0).  Each
# entry holds a hash of the sources the kernel was built from when the
# counters were taken; once those sources change the figure no longer describes
# the kernel and the traffic is reported as null.
FETCH_SCALE, WRITE_SCALE = 2.0, 1.0
COUNTERS = {
    ("prefill_32k", "sparse_mla_kernel"): {
        "sources": ("sparse_mla.hip", "dsa_device.h", "kernels.h"),
        "sha256_16": "d6ff1a9654508436", "fetch_kib": 11540942, "write_kib": 4342829},
    ("prefill_32k", "indexer_prefill_kernel<cand>"): {
        "sources": ("indexer.hip", "indexer_core.h", "dsa_device.h", "kernels.h"),
        "sha256_16": "57034646161a94bc", "fetch_kib": 208660, "write_kib": 838595},
    ("prefill_4k", "sparse_mla_kernel"): {
        "sources": ("sparse_mla.hip", "dsa_device.h", "kernels.h"),
        "sha256_16": "d6ff1a9654508436", "fetch_kib": 475718, "write_kib": 542843},
    ("decode_64k", "indexer_decode_kernel<cand>"): {
        "sources": ("indexer.hip", "indexer_core.h", "dsa_device.h", "kernels.h"),
        "sha256_16": "57034646161a94bc", "fetch_kib": 288538, "write_kib": 2537},
    ("decode_64k", "sparse_mla_kernel"): {
        "sources": ("sparse_mla.hip", "dsa_device.h", "kernels.h"),
        "sha256_16": "d6ff1a9654508436", "fetch_kib": 79250, "write_kib": 33922},
    ("chunked_128k", "indexer_prefill_kernel<cand>"): {
        "sources": ("indexer.hip", "indexer_core.h", "dsa_device.h", "kernels.h"),
        "sha256_16": "57034646161a94bc", "fetch_kib": 206919, "write_kib": 282724},
    ("chunked_128k", "sparse_mla_kernel"): {
        "sources": ("sparse_mla.hip", "dsa_device.h", "kernels.h"),
        "sha256_16": "d6ff1a9654508436", "fetch_kib": 3980437, "write_kib": 542764},
    ("short_prefill_2k", "sparse_mla_kernel"): {
        "sources": ("sparse_mla.hip", "dsa_device.h", "kernels.h"),
        "sha256_16": "d6ff1a9654508436", "fetch_kib": 192795, "write_kib": 271420},
    ("indexer_kl_32k", "indexer_kl_kernel"): {
        "sources": ("indexer_kl.hip", "dsa_device.h", "kernels.h"),
        "sha256_16": "6597be1718ec62a9", "fetch_kib": 21677312, "write_kib": 1361},
    # the whole backward (its 10 kernels, 8 row chunks), summed per call
    ("sparse_bwd_32k", "dsa_sparse_mla_bwd"): {
        "sources": ("sparse_mla_bwd.hip", "dsa_device.h", "kernels.h"),
        "sha256_16": "ae1df37de268b0aa", "fetch_kib": 93224874, "write_kib": 120111233},
    ("quant_append_32k", "quant_groups_kernel<8192,256>"): {
        "sources": ("quant.hip", "dsa_device.h", "kernels.h"),
        "sha256_16": "67a99849d77975ae", "fetch_kib": 524402, "write_kib": 270336},
}

def measured_traffic(workload, kernel):
    """Scaled FETCH+WRITE bytes per launch, or None when no counters were taken
    for this kernel and workload or its sources have changed since."""
    import hashlib
    c = COUNTERS.get((workload, kernel))
    if c is None:
        return None
    h = hashlib.sha256()
    for f in c["sources"]:
        with open(os.path.join(ROOT, "sparse_attention_16_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest()[:16] != c["sha256_16"]:
        return None
    return {"fetch": c["fetch_kib"] * 1024 * FETCH_SCALE, "write": c["write_kib"] * 1024 * WRITE_SCALE}


# ----------------------------------------------------------------- accounting

def visible_counts(cu_q, cu_kv, pos0):
    """Visible keys per query row: min(position + 1, context length)."""
    cu_q, cu_kv, pos0 = np.asarray(cu_q), np.asarray(cu_kv), np.asarray(pos0)
    out = []
    for b in range(len(pos0)):
        nq = int(cu_q[b + 1] - cu_q[b])
        ctx = int(cu_kv[b + 1] - cu_kv[b])
        pos = int(pos0[b]) + np.arange(nq, dtype=np.int64)
        out.append(np.clip(np.minimum(pos + 1, ctx), 0, None))
    return np.concatenate(out) if out else np.zeros(0, np.int64)


def indexer_flops(nvis):
    """FP8 MFMA flops of the index score: 2*HI*DI per visible (query, key) pair."""
    return 2.0 * HI * DI * float(np.sum(nvis))


def mla_flops(nvis, k):
    """bf16 MFMA flops of sparse MQA attention: per selected (query, key) pair,
    H heads x (2*D for q.k + 2*Dv for p.v)."""
    return float(np.sum(np.minimum(nvis, k))) * H * 2.0 * (D + DV)


def dense_mla_flops(nvis):
    return float(np.sum(nvis)) * H * 2.0 * (D + DV)


def indexer_bytes(nvis, ctx_total, T):
    """Algorithmic HBM bytes of the indexer: every cached key (128 code bytes +
    4 scale bytes) and every query row (64x128 codes, 64 scales, 64 weights) read
    once, one fp32 score written per visible pair."""
    return ctx_total * (DI + 4) + T * (HI * DI + HI * 8) + 4.0 * float(np.sum(nvis))


def mla_bytes(nvis, k, T, N=None):
    """Algorithmic HBM bytes of sparse MLA: q + out + idx + lse, plus the latent
    rows.  Without N every selected 1152-byte row is counted (the decode regime,
    where rows are not shared between queries); with N each of the N cached rows
    is counted once (the least any prefill schedule can read)."""
    rows = float(np.sum(np.minimum(nvis, k))) if N is None else min(float(N), float(np.sum(np.minimum(nvis, k))))
    return rows * D * 2 + T * (H * D * 2 + H * DV * 2 + k * 4 + H * 4)


# ------------------------------------------------------------------ workloads

def make_workload(name):
    import synth
    if name == "prefill_32k":
        return synth.prefill(32768), "prefill"
    if name == "prefill_4k":
        return synth.prefill(4096), "prefill"
    if name == "decode_64k":
        return synth.decode(64), "decode"
    if name == "chunked_128k":
        return synth.chunked_prefill(4096, 131072), "prefill"
    if name == "short_prefill_2k":
        # every row sees at most k keys: the fused entry runs the short-sequence mode
        return synth.prefill(2048, seed=SEED_SHORT), "prefill"
    raise SystemExit(f"unknown workload {name}")


def cpu_baseline(wl, target_s=15.0):
    """Oracle (indexer -> top-k -> exact attention) on evenly spaced query rows,
    sized to roughly `target_s` seconds of wall time on this host."""
    import oracle
    b = wl.batch
    T = b.T

    def run(rows):
        inp = wl.sampled_host(rows)
        t0 = time.perf_counter()
        s = oracle.indexer(b.cu_q, b.cu_kv, b.pos0, inp.qi, inp.qi_scale, inp.w, inp.ki,
                           inp.ki_scale, rows=rows)
        idx = oracle.topk(b.cu_q, b.cu_kv, b.pos0, s, wl.k, rows=rows)
        oracle.sparse_attn(b.cu_q, b.cu_kv, b.pos0, inp.q, inp.kv, idx, wl.Dv, wl.scale, rows=rows)
        return time.perf_counter() - t0

    threads = oracle.num_threads()
    probe = np.unique(np.linspace(0, T - 1, min(T, max(threads, 8))).astype(np.int64))
    dt = run(probe)
    per_row = dt / len(probe)
    n = int(min(T, max(len(probe), math.floor(target_s / max(per_row, 1e-6)))))
    rows = np.unique(np.linspace(0, T - 1, n).astype(np.int64))
    dt = run(rows)
    return {"value": len(rows) / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(rows)} query rows evenly spaced over all {T} rows of the same "
                      f"workload (full indexer row, top-{wl.k}, exact attention per row), "
                      f"{dt:.1f} s wall"}


# ---------------------------------------------------------- quantise + append

KL_METRIC = "indexer KL loss tokens/s (sparse stage over the top-2048 selection), 32K prefill"


def kl_bench(args, dsa):
    """One step = the indexer KL loss of every row of a 32K prefill in the
    sparse training stage: the target (the attention's probabilities over the
    2048 selected rows, summed over the 128 heads, L1-normalised) against the
    softmax of the index scores.  Its inputs (index scores, selection,
    attention lse) come from the library's own forward, run once before the
    timed region; q and the latent cache are the prefill_32k inputs."""
    import torch
    say = lambda *a: print(*a, file=sys.stderr, flush=True)  # noqa: E731
    wl, _ = make_workload("prefill_32k")
    b = wl.batch
    t0 = time.time()
    dev = wl.device("cuda")
    batch = dsa.Batch.from_host(b.cu_q, b.cu_kv, b.pos0)
    ld = ((b.max_kv + 63) // 64) * 64
    scores = torch.empty((b.T, ld), dtype=torch.float32, device="cuda")
    idx = torch.empty((b.T, wl.k), dtype=torch.int32, device="cuda")
    out = torch.empty((b.T, H, DV), dtype=torch.int16, device="cuda")
    lse = torch.empty((b.T, H), dtype=torch.float32, device="cuda")
    dsa.indexer_scores(batch, dev["qi"], dev["qs"], dev["w"], dev["ki"], dev["ks"], scores)
    dsa.topk(batch, scores, wl.k, idx)
    dsa.sparse_mla_fwd(batch, dev["q"], dev["kv"], idx, wl.scale, out, lse)
    del out
    kl = torch.empty(b.T, dtype=torch.float32, device="cuda")
    ws = torch.empty(max(1, dsa.workspace_size(dsa.WS_INDEXER_KL, batch, wl.k)), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    say(f"[bench] workload indexer_kl_32k: T={b.T} k={wl.k}; inputs and forward ready ({time.time() - t0:.1f} s)")

    def step():
        dsa.indexer_kl_fwd(batch, dev["q"], dev["kv"], lse, wl.scale, scores, kl, idx=idx, ws=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t1
    ms_per_step = elapsed * 1e3 / args.steps
    tokens_per_s = b.T * args.steps / elapsed
    say(f"[bench] {args.steps} steps: {ms_per_step:.3f} ms/step, {tokens_per_s:,.0f} tokens/s")

    nvis = visible_counts(b.cu_q, b.cu_kv, b.pos0)
    flops = float(np.sum(np.minimum(nvis, wl.k))) * H * 2.0 * D      # the logits of the selected pairs
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.kernel_reps)]
    for e0, e1 in evs:
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    kms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs]))
    achieved = flops / (kms * 1e-3) / 1e12
    roof = {"kernel": "indexer_kl_kernel", "bound": "mfma", "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": None, "avg_ms": round(kms, 4), "algorithmic_flops": flops}
    tr = measured_traffic("indexer_kl_32k", "indexer_kl_kernel")
    if tr is not None:
        roof["traffic"] = round(tr["fetch"] + tr["write"])
        roof["traffic_unit"] = "bytes/launch (FETCH_SIZE+WRITE_SIZE, copy-calibrated)"
        roof["traffic_fetch"], roof["traffic_write"] = round(tr["fetch"]), round(tr["write"])
    say(f"[bench] indexer_kl_kernel: {kms:.3f} ms/launch, {achieved:.1f} TFLOP/s ({100 * roof['frac']:.1f}% of peak)")

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        say("[bench] timing the CPU oracle on a sample of the workload ...")
        threads = oracle.num_threads()

        def run(n):
            # the loss's inputs for the sampled rows from the oracle itself (untimed)
            rows = np.unique(np.linspace(0, b.T - 1, n).astype(np.int64))
            inp = wl.sampled_host(rows)
            s_rows = oracle.indexer(b.cu_q, b.cu_kv, b.pos0, inp.qi, inp.qi_scale, inp.w, inp.ki, inp.ki_scale,
                                    rows=rows)
            i_rows = oracle.topk(b.cu_q, b.cu_kv, b.pos0, s_rows, wl.k, rows=rows)
            t2 = time.perf_counter()
            oracle.indexer_kl(b.cu_q, b.cu_kv, b.pos0, inp.q, inp.kv, wl.scale, s_rows, idx=i_rows, rows=rows)
            return len(rows), time.perf_counter() - t2
        n0, dt = run(16)
        # (the oracle's scores and selection for a sampled row cost more than its loss: at most 1024 rows)
        n = int(min(b.T, 1024, max(16, args.cpu_seconds / max(dt / n0, 1e-9))))
        n, dt = run(n)
        cpu = {"value": n / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
               "sample": f"{n} query rows evenly spaced over the {b.T} of the workload (exact per-head softmax, "
                         f"head sum, KL over the 2048 selected keys; the oracle's index scores and selection "
                         f"for those rows made first, untimed), {dt:.1f} s wall"}
        say(f"[bench] CPU oracle: {cpu['value']:.2f} tokens/s on {threads} threads")

    cfg = {"workload": "indexer_kl_32k", "batch": b.B, "query_tokens": b.T, "cache_rows": b.N, "topk": wl.k,
           "heads": H, "d_qk": D, "entry": "dsa_indexer_kl_fwd (sparse stage)"}
    line = {"metric": KL_METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic", "config": cfg, "roofline": roof, "cpu_baseline": cpu}
    print(json.dumps(line), flush=True)
    return 0


TOPK_METRIC = "standalone top-2048 rows/s over a 32K prefill's index scores (dsa_topk)"


def topk_bench(args, dsa):
    """One step = dsa_topk over the index scores of a 32K prefill (every row
    of the causal 32768 x 32768 score matrix, the three-step API's select).
    The scores come from dsa_indexer_scores on the prefill_32k inputs, run
    once before the timed region."""
    import torch
    say = lambda *a: print(*a, file=sys.stderr, flush=True)  # noqa: E731
    wl, _ = make_workload("prefill_32k")
    b = wl.batch
    t0 = time.time()
    dev = wl.device("cuda")
    batch = dsa.Batch.from_host(b.cu_q, b.cu_kv, b.pos0)
    ld = ((b.max_kv + 63) // 64) * 64
    scores = torch.empty((b.T, ld), dtype=torch.float32, device="cuda")
    idx = torch.empty((b.T, wl.k), dtype=torch.int32, device="cuda")
    dsa.indexer_scores(batch, dev["qi"], dev["qs"], dev["w"], dev["ki"], dev["ks"], scores)
    for key in ("qi", "qs", "w", "q", "kv"):
        dev.pop(key, None)
    ws = torch.empty(max(1, dsa.workspace_size(dsa.WS_TOPK, batch, wl.k)), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    say(f"[bench] workload topk_32k: T={b.T} k={wl.k}; index scores ready ({time.time() - t0:.1f} s)")

    def step():
        dsa.topk(batch, scores, wl.k, idx, ws=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t1
    ms_per_step = elapsed * 1e3 / args.steps
    rows_per_s = b.T * args.steps / elapsed
    say(f"[bench] {args.steps} steps: {ms_per_step:.4f} ms/step, {rows_per_s:,.0f} rows/s")

    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(max(20, args.profile_reps))]
    for e0, e1 in evs:
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    times = [e0.elapsed_time(e1) for e0, e1 in evs]
    nvis = visible_counts(b.cu_q, b.cu_kv, b.pos0)
    roof = kernel_roof("topk_chunk_kernel", wl, "prefill", nvis, float(np.mean(times)), float(np.median(times)))
    roof["traffic"] = None
    roof["chosen_by"] = "the entry's only launch (one 32768-column chunk per row)"
    say(f"[bench] topk_chunk_kernel: {roof['avg_ms']:.4f} ms mean, {roof['median_ms']:.4f} median  "
        f"{roof['achieved']} GB/s ({100 * roof['frac']:.1f}% of peak, target {100 * roof['target_frac']:.0f}%)")
    bad = dsa.check_selection(batch, idx)
    assert bad == 0, f"{bad} rows break the selection contract"

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        say("[bench] timing the CPU oracle on a sample of the workload ...")
        threads = oracle.num_threads()
        rows_all = np.linspace(0, b.T - 1, 4096).astype(np.int64)
        host = scores[torch.from_numpy(rows_all).cuda()].cpu().numpy()

        def run(n):
            sel = np.unique(np.linspace(0, len(rows_all) - 1, n).astype(np.int64))
            rows = rows_all[sel]
            s_rows = np.ascontiguousarray(host[sel])
            t2 = time.perf_counter()
            oracle.topk(b.cu_q, b.cu_kv, b.pos0, s_rows, wl.k, rows=rows)
            return len(rows), time.perf_counter() - t2
        n0, dt = run(64)
        n = int(min(len(rows_all), max(64, args.cpu_seconds / max(dt / n0, 1e-9))))
        n, dt = run(n)
        cpu = {"value": n / dt, "unit": "rows/s", "cores": threads, "kind": "oracle",
               "sample": f"{n} query rows evenly spaced over the {b.T} of the workload (the GPU's index "
                         f"scores of those rows copied to the host first, untimed), {dt:.1f} s wall"}
        cpu.update(cpu_info())
        say(f"[bench] CPU oracle: {cpu['value']:.2f} rows/s on {threads} threads")

    cfg = {"workload": "topk_32k", "batch": b.B, "query_tokens": b.T, "max_context": b.max_kv, "topk": wl.k,
           "score_columns": ld, "entry": "dsa_topk (three-step API)"}
    line = {"metric": TOPK_METRIC, "value": round(rows_per_s, 1), "unit": "rows/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp32 (u32 keys)",
            "data": "synthetic", "config": cfg, "roofline": roof, "cpu_baseline": cpu}
    if not args.no_peaks:
        peaks = attainable_peaks(dsa)
        line["attainable_peaks"] = peaks
        attach_attainable(roof, peaks)
    print(json.dumps(line), flush=True)
    return 0


BWD_METRIC = "sparse MLA backward tokens/s (dq and dkv over the top-2048 selection), 32K prefill"
SEED_DOUT = 0xD5A8         # seed of the attention output gradient


def bwd_bench(args, dsa):
    """One step = the backward of the sparse attention of a 32K prefill (dq of
    every row, dkv of the latent cache) for a seeded bf16 output gradient.
    The selection, out and lse come from the library's own forward, run once
    before the timed region; q and the latent cache are the prefill_32k inputs."""
    import torch
    say = lambda *a: print(*a, file=sys.stderr, flush=True)  # noqa: E731
    wl, _ = make_workload("prefill_32k")
    b = wl.batch
    t0 = time.time()
    dev = wl.device("cuda")
    batch = dsa.Batch.from_host(b.cu_q, b.cu_kv, b.pos0)
    fargs = dsa.fwd_args(batch, dev["qi"], dev["qs"], dev["w"], dev["ki"], dev["ks"], dev["q"], dev["kv"], wl.k,
                         wl.scale)
    out = torch.empty((b.T, H, DV), dtype=torch.int16, device="cuda")
    lse = torch.empty((b.T, H), dtype=torch.float32, device="cuda")
    idx = torch.empty((b.T, wl.k), dtype=torch.int32, device="cuda")
    dsa.prefill_fwd(fargs, batch, out, lse, idx)
    g = torch.Generator("cuda").manual_seed(SEED_DOUT)
    dout = torch.randn((b.T, H, DV), dtype=torch.float32, device="cuda", generator=g).to(torch.bfloat16) \
        .view(torch.int16)
    dq = torch.empty((b.T, H, D), dtype=torch.float32, device="cuda")
    dkv = torch.empty((b.N, D), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(1, dsa.workspace_size(dsa.WS_SPARSE_MLA_BWD, batch, wl.k)), dtype=torch.uint8,
                     device="cuda")
    torch.cuda.synchronize()
    say(f"[bench] workload sparse_bwd_32k: T={b.T} k={wl.k}; inputs and forward ready ({time.time() - t0:.1f} s)")

    def step():
        dsa.sparse_mla_bwd(batch, dev["q"], dev["kv"], idx, wl.scale, out, lse, dout, dq, dkv, ws=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t1
    ms_per_step = elapsed * 1e3 / args.steps
    tokens_per_s = b.T * args.steps / elapsed
    say(f"[bench] {args.steps} steps: {ms_per_step:.3f} ms/step, {tokens_per_s:,.0f} tokens/s")

    # algorithmic work of the whole backward: per selected (row, key) pair and head,
    # the logits (576), dP (512), dq (576), the key side (576) and the value side (512)
    nvis = visible_counts(b.cu_q, b.cu_kv, b.pos0)
    pairs = float(np.sum(np.minimum(nvis, wl.k)))
    flops = pairs * H * 2.0 * (D + DV + D + D + DV)
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.kernel_reps)]
    for e0, e1 in evs:
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    kms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs]))
    achieved = flops / (kms * 1e-3) / 1e12
    roof = {"kernel": "dsa_sparse_mla_bwd (all launches)", "bound": "mfma",
            "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None, "avg_ms": round(kms, 4),
            "algorithmic_flops": flops}
    tr = measured_traffic("sparse_bwd_32k", "dsa_sparse_mla_bwd")
    if tr is not None:
        roof["traffic"] = round(tr["fetch"] + tr["write"])
        roof["traffic_unit"] = "bytes/call, all kernels of the backward (FETCH_SIZE+WRITE_SIZE, copy-calibrated)"
        roof["traffic_fetch"], roof["traffic_write"] = round(tr["fetch"]), round(tr["write"])
    say(f"[bench] backward: {kms:.3f} ms/launch, {achieved:.1f} TFLOP/s ({100 * roof['frac']:.1f}% of peak)")

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        say("[bench] timing the CPU oracle on a sample of the workload ...")
        threads = oracle.num_threads()

        def run(n):
            # the backward's inputs for the sampled rows from the oracle itself (untimed)
            rows = np.unique(np.linspace(0, b.T - 1, n).astype(np.int64))
            inp = wl.sampled_host(rows)
            s_rows = oracle.indexer(b.cu_q, b.cu_kv, b.pos0, inp.qi, inp.qi_scale, inp.w, inp.ki, inp.ki_scale,
                                    rows=rows)
            i_rows = oracle.topk(b.cu_q, b.cu_kv, b.pos0, s_rows, wl.k, rows=rows)
            gd = np.zeros((b.T, H, DV), np.float32)
            gd[rows] = np.random.default_rng(SEED_DOUT).standard_normal((len(rows), H, DV)).astype(np.float32)
            t2 = time.perf_counter()
            oracle.sparse_attn_bwd(b.cu_q, b.cu_kv, b.pos0, inp.q, inp.kv, gd, i_rows, wl.Dv, wl.scale, rows=rows)
            return len(rows), time.perf_counter() - t2
        n0, dt = run(16)
        n = int(min(b.T, 512, max(16, args.cpu_seconds / max(dt / n0, 1e-9))))
        n, dt = run(n)
        cpu = {"value": n / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
               "sample": f"{n} query rows evenly spaced over the {b.T} of the workload (exact softmax backward, "
                         f"dq and the rows' dkv contributions over the 2048 selected keys; the oracle's scores and "
                         f"selection for those rows made first, untimed), {dt:.1f} s wall"}
        say(f"[bench] CPU oracle: {cpu['value']:.2f} tokens/s on {threads} threads")

    cfg = {"workload": "sparse_bwd_32k", "batch": b.B, "query_tokens": b.T, "cache_rows": b.N, "topk": wl.k,
           "heads": H, "d_qk": D, "d_v": DV, "entry": "dsa_sparse_mla_bwd"}
    line = {"metric": BWD_METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic", "config": cfg, "roofline": roof, "cpu_baseline": cpu}
    print(json.dumps(line), flush=True)
    return 0


QUANT_METRIC = "FP8 quantise + cache append tokens/s (indexer queries and keys, latent rows), 32K prefill"


def quant_append_bench(args, dsa):
    """One step = the 32768 new tokens of a 32K prefill: their indexer queries
    [T, 64, 128] fp32 quantised to E4M3FN with one scale per token, their
    indexer keys [T, 128] fp32 quantised (one scale per key) and appended to the
    FP8 key cache, their bf16 latent rows [T, 576] appended to the latent cache.
    Inputs are seeded standard normals (the distribution the index-score
    inputs are drawn from), resident in HBM."""
    import torch
    say = lambda *a: print(*a, file=sys.stderr, flush=True)  # noqa: E731
    T = N = 32768
    g = torch.Generator("cuda").manual_seed(SEED_QUANT)
    q = torch.randn((T, HI, DI), dtype=torch.float32, device="cuda", generator=g)
    k_new = torch.randn((T, DI), dtype=torch.float32, device="cuda", generator=g)
    kv_new = torch.randn((T, D), dtype=torch.float32, device="cuda", generator=g).to(torch.bfloat16).view(torch.int16)
    dst = torch.arange(T, dtype=torch.int64, device="cuda")
    q_fp8 = torch.empty((T, HI, DI), dtype=torch.uint8, device="cuda")
    q_scale = torch.empty((T, HI), dtype=torch.float32, device="cuda")
    k_fp8 = torch.empty((N, DI), dtype=torch.uint8, device="cuda")
    k_scale = torch.empty((N,), dtype=torch.float32, device="cuda")
    kv = torch.empty((N, D), dtype=torch.int16, device="cuda")
    torch.cuda.synchronize()
    say(f"[bench] workload quant_append_32k: T={T} tokens, cache rows N={N}")

    def step():
        dsa.quantize_queries(q, q_fp8, q_scale)
        dsa.append_cache(k_new, kv_new, dst, k_fp8, k_scale, kv)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    tokens_per_s = T * args.steps / elapsed
    say(f"[bench] {args.steps} steps: {ms_per_step:.3f} ms/step, {tokens_per_s:,.0f} tokens/s")

    # dominant kernel: the query quantiser (4 B read + 1 B written per value, 64 scales per token)
    stream = torch.cuda.current_stream()
    nbytes = T * HI * DI * (4 + 1) + T * HI * 4
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.kernel_reps)]
    for e0, e1 in evs:
        e0.record(stream)
        dsa.quantize_queries(q, q_fp8, q_scale)
        e1.record(stream)
    torch.cuda.synchronize()
    kms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs]))
    achieved = nbytes / (kms * 1e-3) / 1e9
    roof = {"kernel": "quant_groups_kernel<8192,256>", "bound": "hbm", "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": None, "avg_ms": round(kms, 4), "algorithmic_bytes": nbytes}
    tr = measured_traffic("quant_append_32k", "quant_groups_kernel<8192,256>")
    if tr is not None:
        roof["traffic"] = round(tr["fetch"] + tr["write"])
        roof["traffic_unit"] = "bytes/launch (FETCH_SIZE+WRITE_SIZE, copy-calibrated)"
        roof["traffic_fetch"], roof["traffic_write"] = round(tr["fetch"]), round(tr["write"])
    say(f"[bench] query quantiser: {kms:.3f} ms/launch, {achieved:.1f} GB/s ({100 * roof['frac']:.1f}% of peak)")

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        say("[bench] timing the CPU oracle on a sample of the workload ...")
        threads = oracle.num_threads()

        def run(n):
            rows = np.unique(np.linspace(0, T - 1, n).astype(np.int64))
            x = q[torch.from_numpy(rows).cuda()].reshape(len(rows), HI * DI).cpu().numpy()
            kx = k_new[torch.from_numpy(rows).cuda()].cpu().numpy()
            t1 = time.perf_counter()
            oracle.quant_rows(x)
            oracle.quant_rows(kx)
            return len(rows), time.perf_counter() - t1
        n0, dt = run(64)
        n = int(min(T, max(64, args.cpu_seconds / max(dt / n0, 1e-9))))
        n, dt = run(n)
        cpu = {"value": n / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
               "sample": f"{n} tokens evenly spaced over the {T} of the workload (query and key "
                         f"quantisation; the latent copy is not timed), {dt:.1f} s wall"}
        say(f"[bench] CPU oracle: {cpu['value']:.2f} tokens/s on {threads} threads")

    cfg = {"workload": "quant_append_32k", "query_tokens": T, "cache_rows": N, "indexer_heads": HI,
           "indexer_dim": DI, "d_latent": D, "entry": "dsa_quantize_queries + dsa_append_cache"}
    line = {"metric": QUANT_METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32->e4m3",
            "data": "synthetic", "config": cfg, "roofline": roof, "cpu_baseline": cpu}
    print(json.dumps(line), flush=True)
    return 0


# ---------------------------------------------------------------------- bench

def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="headline",
                    choices=["headline", "prefill_32k", "prefill_4k", "decode_64k", "chunked_128k",
                             "quant_append_32k", "short_prefill_2k", "indexer_kl_32k", "sparse_bwd_32k",
                             "topk_32k"],
                    help="headline (default): prefill_32k with the decode_64k figures nested in the same line")
    ap.add_argument("--decode-steps", type=int, default=200,
                    help="timed steps of the nested decode_64k figures (at least --steps)")
    ap.add_argument("--profile-reps", type=int, default=20,
                    help="calls timed per kernel with HIP events (at least 20; 0: none, for counter runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--kernel-reps", type=int, default=5,
                    help="timed launches of the dominant kernel")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the attainable-peak loops (dsa_measure_peaks) after the workload")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 3 times (reference "
                         "for scaling the FETCH_SIZE / WRITE_SIZE counters) and exit")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py: the DSA path runs on a single GPU; --gpus {args.gpus} is not "
              "supported (no multi-GPU sharding is implemented).", file=sys.stderr)
        return 2

    import torch

    torch.cuda.set_device(0)
    if args.copy_calibration:
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n}))
        return 0
    import sparse_attention_16_amd as dsa

    if args.workload == "quant_append_32k":
        return quant_append_bench(args, dsa)
    if args.workload == "topk_32k":
        return topk_bench(args, dsa)
    if args.workload == "indexer_kl_32k":
        return kl_bench(args, dsa)
    if args.workload == "sparse_bwd_32k":
        return bwd_bench(args, dsa)
    if args.workload == "headline":
        line = fwd_bench(args, dsa, "prefill_32k", args.steps, args.warmup)
        dec_steps = max(args.steps, args.decode_steps)
        dec = fwd_bench(args, dsa, "decode_64k", dec_steps, max(args.warmup, 10))
        line["decode_64k"] = {k: dec[k] for k in ("value", "unit", "steps", "warmup", "ms_per_step", "timing",
                                                  "config", "roofline", "kernels", "cpu_baseline") if k in dec}
        line["decode_64k"]["tokens_per_s"] = dec["value"]
    else:
        line = fwd_bench(args, dsa, args.workload, args.steps, args.warmup)
    if not args.no_peaks and line.get("roofline"):
        peaks = attainable_peaks(dsa)
        line["attainable_peaks"] = peaks
        for part in (line, line.get("decode_64k")):
            if part:
                attach_attainable(part["roofline"], peaks)
                for r in part.get("kernels", []):
                    attach_attainable(r, peaks)
    print(json.dumps(line), flush=True)
    return 0


def attainable_peaks(dsa):
    """What this GPU reaches on the instructions the rooflines price
    (dsa_measure_peaks: MFMA loops, a streaming read and copy over 2 GiB),
    next to the spec-sheet peaks the fractions divide by."""
    import torch
    buf = torch.empty(2 << 30, dtype=torch.uint8, device="cuda")
    p = dsa.measure_peaks(buf)
    del buf
    say = lambda *a: print(*a, file=sys.stderr, flush=True)  # noqa: E731
    say(f"[bench] attainable on this GPU: bf16 MFMA {p['bf16_tflops']:.0f} TFLOP/s "
        f"({100 * p['bf16_tflops'] / PEAK_BF16_TFLOPS:.0f}% of the spec sheet), FP8 MFMA {p['fp8_tflops']:.0f} "
        f"({100 * p['fp8_tflops'] / PEAK_FP8_TFLOPS:.0f}%), HBM read {p['hbm_read_gbs']:.0f} GB/s "
        f"({100 * p['hbm_read_gbs'] / PEAK_HBM_GBS:.0f}%), copy {p['hbm_copy_gbs']:.0f} GB/s")
    return {k: round(v, 1) for k, v in p.items()} | {
        "note": "best of 3 runs: 8 independent MFMA chains per wave, 16 waves per compute unit; non-temporal "
                "16-byte streaming read of 2 GiB and copy of 1 GiB (read + write bytes)"}


def attach_attainable(roof, peaks):
    """The roofline's rate against what this GPU attains for its bound: the
    MFMA loop of its own data type, or the better of the streaming read and copy."""
    if roof.get("bound") == "mfma":
        a = peaks["fp8_tflops"] if roof.get("peak") == PEAK_FP8_TFLOPS else peaks["bf16_tflops"]
    elif roof.get("bound") == "hbm":
        a = max(peaks["hbm_read_gbs"], peaks["hbm_copy_gbs"])
    else:
        return
    if "achieved" not in roof:
        return
    roof["attainable_peak"] = round(a, 1)
    roof["frac_attainable"] = round(roof["achieved"] / a, 4) if a > 0 else None


# ------------------------------------------------------ fused forward (A1-A9)

def cpu_info():
    """The host the CPU baseline ran on: model, logical CPUs, affinity, OpenMP setting."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        aff = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        aff = None
    return {"cpu_model": model, "nproc": os.cpu_count(), "affinity_cpus": aff,
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS")}


def sampled_pairs(batch, k):
    """(query, key) pairs the threshold sample scores: per block of 16 query
    rows of a sequence whose longest row sees n > 4096 (and > k) keys, the keys
    o + i * (n // m), i < m = clamp(n // 32, 512, 1024), that each row sees
    (the sample kernel's grid, offset hashed from the block and the sequence)."""
    cu_q, cu_kv, pos0 = np.asarray(batch.cu_q), np.asarray(batch.cu_kv), np.asarray(batch.pos0)
    total = 0
    for sq in range(len(pos0)):
        nq = int(cu_q[sq + 1] - cu_q[sq])
        ctx = int(cu_kv[sq + 1] - cu_kv[sq])
        nv = np.clip(np.minimum(int(pos0[sq]) + np.arange(nq) + 1, ctx), 0, None)
        for blk in range(0, nq, 16):
            rows = nv[blk:blk + 16]
            n_hi = int(rows.max())
            if n_hi <= 4096 or n_hi <= k:
                continue
            m = min(max(n_hi // 32, 512), 1024)
            stride = n_hi // m
            o = (((blk // 16) * 2654435761 + sq * 40503) & 0xFFFFFFFF) % stride
            total += int(np.sum(np.clip(-(-(rows - o) // stride), 0, m)))
    return total


def scored_rows(batch, k):
    """Visible counts of the rows the candidate indexer scores: every row of a
    16-row block whose longest row sees more than k keys (blocks that see at
    most k keys need no scores; prefill layout)."""
    cu_q, cu_kv, pos0 = np.asarray(batch.cu_q), np.asarray(batch.cu_kv), np.asarray(batch.pos0)
    out = []
    for sq in range(len(pos0)):
        nq = int(cu_q[sq + 1] - cu_q[sq])
        ctx = int(cu_kv[sq + 1] - cu_kv[sq])
        nv = np.clip(np.minimum(int(pos0[sq]) + np.arange(nq) + 1, ctx), 0, None)
        for blk in range(0, nq, 16):
            rows = nv[blk:blk + 16]
            if rows.max() > k:
                out.append(rows)
    return np.concatenate(out) if out else np.zeros(0, np.int64)


def kernel_roof(name, wl, entry, nvis, ms_mean, ms_median, splits=1, items=-1):
    """Roofline of one kernel of the fused forward: its bound, algorithmic work
    per launch (flops or HBM bytes, as stated per kernel below), achieved rate
    on the mean launch time, fraction of the MI355X peak and the target."""
    b = wl.batch
    k, T = wl.k, b.T
    long_rows = nvis > k
    if name in ("indexer_sample_kernel", "indexer_sample_row_kernel"):
        bound, work = "mfma", 2.0 * HI * DI * sampled_pairs(b, k)   # fp8 flops of the sampled pairs
        peak, unit, target = PEAK_FP8_TFLOPS, "TFLOP/s", 0.5
    elif name == "indexer_prefill_kernel<cand>":
        bound, work = "mfma", indexer_flops(scored_rows(b, k))     # 2*64*128 fp8 flops per scored visible pair
        peak, unit, target = PEAK_FP8_TFLOPS, "TFLOP/s", 0.5
    elif name == "indexer_decode_kernel<cand>":
        # keys (128 code bytes + 4 scale bytes) of rows that see more than k, their query rows
        work = (DI + 4) * float(np.sum(nvis[long_rows])) + float(np.sum(long_rows)) * (HI * DI + HI * 8)
        bound, peak, unit, target = "hbm", PEAK_HBM_GBS, "GB/s", 0.5
    elif name in ("cand_select_wave_kernel", "cand_select_wave_contig_kernel"):
        # candidate keys read, the selected positions read, idx written
        work = 4.0 * max(items, 0) + 8.0 * k * T
        bound, peak, unit, target = "hbm", PEAK_HBM_GBS, "GB/s", 0.6
    elif name == "indexer_prefill_kernel":
        bound, work = "mfma", indexer_flops(nvis)            # 2*64*128 fp8 flops per visible pair
        peak, unit, target = PEAK_FP8_TFLOPS, "TFLOP/s", 0.5
    elif name == "indexer_decode_kernel":
        bound, work = "hbm", indexer_bytes(nvis, b.N, T)     # keys + scales + queries read, scores written
        peak, unit, target = PEAK_HBM_GBS, "GB/s", 0.5
    elif name == "topk_chunk_kernel":
        nch = np.ceil(nvis / 32768.0)
        # scores of rows longer than k read once, idx written; chunked rows write (key, position) candidates
        work = 4.0 * float(np.sum(nvis[long_rows])) + 4.0 * k * T + 8.0 * k * float(np.sum(nch[nvis > 32768]))
        bound, peak, unit, target = "hbm", PEAK_HBM_GBS, "GB/s", 0.6
    elif name == "topk_merge_kernel":
        nch = np.ceil(nvis / 32768.0)
        work = 8.0 * k * float(np.sum(nch[nvis > 32768])) + 4.0 * k * float(np.sum(nvis > 32768))
        bound, peak, unit, target = "hbm", PEAK_HBM_GBS, "GB/s", 0.6
    elif name == "sparse_mla_kernel" and splits == 1:
        bound, work = "mfma", mla_flops(nvis, k)              # 128 heads x 2 x (576 + 512) per selected pair
        peak, unit, target = PEAK_BF16_TFLOPS, "TFLOP/s", 0.5
    elif name == "sparse_mla_kernel":
        # split-KV (few rows): every selected latent row gathered from HBM, q read, partials written
        work = mla_bytes(nvis, k, T) - T * H * DV * 2 + T * splits * H * (DV * 2 + 4)
        bound, peak, unit, target = "hbm", PEAK_HBM_GBS, "GB/s", 0.6
    elif name == "mla_merge_kernel":
        work = T * splits * H * (DV * 2 + 4) + T * H * (DV * 2 + 4)
        bound, peak, unit, target = "hbm", PEAK_HBM_GBS, "GB/s", 0.6
    elif name == "select_all_visible_kernel":
        work = 4.0 * k * T
        bound, peak, unit, target = "hbm", PEAK_HBM_GBS, "GB/s", 0.6
    else:
        r = {"kernel": name, "avg_ms": round(ms_mean, 4), "median_ms": round(ms_median, 4)}
        if items >= 0:
            r["items"] = items
        return r
    rate = work / (ms_mean * 1e-3) / (1e12 if unit == "TFLOP/s" else 1e9)
    r = {"kernel": name, "bound": bound, "achieved": round(rate, 2), "peak": peak, "unit": unit,
         "frac": round(rate / peak, 4), "target_frac": target, "avg_ms": round(ms_mean, 4),
         "median_ms": round(ms_median, 4)}
    if items >= 0:
        r["items"] = items
    r["algorithmic_flops" if bound == "mfma" else "algorithmic_bytes"] = float(work)
    return r


def fwd_bench(args, dsa, workload, steps, warmup):
    """One fused-forward workload: K timed steps (wall clock, synchronised on
    both sides), then per-kernel HIP-event times over --profile-reps calls of
    the same entry, and the step's event median with and without an Infinity
    Cache flush (a 512 MB write) before each call.  Returns the JSON object."""
    import torch
    say = lambda *a: print(*a, file=sys.stderr, flush=True)  # noqa: E731
    wl, entry = make_workload(workload)
    b = wl.batch
    say(f"[bench] workload {workload}: T={b.T} N={b.N} B={b.B} max_kv={b.max_kv}")
    t0 = time.time()
    dev = wl.device("cuda")
    torch.cuda.synchronize()
    say(f"[bench] inputs generated and resident in HBM ({time.time() - t0:.1f} s)")

    batch = dsa.Batch.from_host(b.cu_q, b.cu_kv, b.pos0)
    fargs = dsa.fwd_args(batch, dev["qi"], dev["qs"], dev["w"], dev["ki"], dev["ks"], dev["q"],
                         dev["kv"], wl.k, wl.scale)
    out = torch.empty((b.T, H, DV), dtype=torch.int16, device="cuda")
    lse = torch.empty((b.T, H), dtype=torch.float32, device="cuda")
    idx = torch.empty((b.T, wl.k), dtype=torch.int32, device="cuda")
    ws_entry = dsa.WS_PREFILL if entry == "prefill" else dsa.WS_DECODE
    ws_bytes = dsa.workspace_size(ws_entry, batch, wl.k)
    ws = torch.empty(max(1, ws_bytes), dtype=torch.uint8, device="cuda")
    fwd = dsa.prefill_fwd if entry == "prefill" else dsa.decode_fwd
    stream = torch.cuda.current_stream()

    def step():
        fwd(fargs, batch, out, lse, idx, ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / steps
    tokens_per_s = b.T * steps / elapsed
    say(f"[bench] {steps} steps: {ms_per_step:.4f} ms/step, {tokens_per_s:,.0f} tokens/s")

    if args.profile_reps == 0:
        # (counter collection: only the K timed steps, no per-kernel legs)
        return {"metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
                "steps": steps, "warmup": warmup, "ms_per_step": round(ms_per_step, 4),
                "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp8+bf16",
                "data": "synthetic", "config": {"workload": workload}, "roofline": None, "cpu_baseline": None}
    # ---- per-kernel times: HIP events around each launch of the same entry, on its stream
    reps = max(20, args.profile_reps)
    per = {}
    items = {}
    order = []
    step_ev = []
    for _ in range(reps):
        tl = dsa.fwd_profile(fargs, batch, out, lse, idx, ws, decode=(entry == "decode"), stream=stream)
        step_ev.append(sum(ms for _, ms, _ in tl))
        for kname, ms, it in tl:
            if kname not in per:
                per[kname] = []
                order.append(kname)
            per[kname].append(ms)
            items[kname] = it
    # the same, each call after a 512 MB write that evicts the Infinity Cache
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    step_cold = []
    for i in range(reps):
        flush.fill_(i & 0xFF)
        torch.cuda.synchronize()
        tl = dsa.fwd_profile(fargs, batch, out, lse, idx, ws, decode=(entry == "decode"), stream=stream)
        step_cold.append(sum(ms for _, ms, _ in tl))
    del flush
    nvis = visible_counts(b.cu_q, b.cu_kv, b.pos0)
    splits = 1
    if entry == "decode" or b.T < 256:
        # split-KV factor the library takes for few rows: one workgroup per compute unit
        ncu = torch.cuda.get_device_properties(0).multi_processor_count
        splits = 1 if b.T >= ncu else min(-(-ncu // b.T), -(-wl.k // 32))
    kernels = [kernel_roof(kn, wl, entry, nvis, float(np.mean(per[kn])), float(np.median(per[kn])), splits,
                           items.get(kn, -1))
               for kn in order]
    dom = max(kernels, key=lambda r: r["avg_ms"])
    roof = dict(dom)
    roof["traffic"] = None
    tr = measured_traffic(workload, dom["kernel"])
    if tr is not None:
        roof["traffic"] = round(tr["fetch"] + tr["write"])
        roof["traffic_unit"] = "bytes/launch (FETCH_SIZE+WRITE_SIZE, copy-calibrated)"
        roof["traffic_fetch"], roof["traffic_write"] = round(tr["fetch"]), round(tr["write"])
    roof["chosen_by"] = "largest mean HIP-event time among the step's kernels"
    for r in kernels:
        tgt = f", target {100 * r['target_frac']:.0f}%" if "frac" in r else ""
        rate = f"{r['achieved']} {r['unit']} ({100 * r['frac']:.1f}% of peak{tgt})" if "frac" in r else ""
        if "items" in r:
            rate += f" [{r['items']} items]"
        say(f"[bench]   {r['kernel']}: {r['avg_ms']:.4f} ms mean, {r['median_ms']:.4f} median  {rate}")
    timing = {"events_reps": reps, "step_ms_median": round(float(np.median(step_ev)), 4),
              "step_ms_median_mall_flushed": round(float(np.median(step_cold)), 4),
              "note": "value uses the wall clock over the K steps; the medians are sums of the per-kernel "
                      "HIP-event intervals of single calls (the flushed one writes 512 MB before each call)"}
    say(f"[bench] event median per step {timing['step_ms_median']} ms, "
        f"after a cache flush {timing['step_ms_median_mall_flushed']} ms")

    three = None
    if b.max_kv <= wl.k:
        # short-sequence mode: the same forward through the three separate steps
        # (indexer -> top-k -> sparse attention over the -1 padded selection)
        ld = ((b.max_kv + 63) // 64) * 64
        scores = torch.empty((b.T, ld), dtype=torch.float32, device="cuda")
        idx3 = torch.empty_like(idx)
        out3, lse3 = torch.empty_like(out), torch.empty_like(lse)
        tws = torch.empty(max(1, dsa.workspace_size(dsa.WS_TOPK, batch, wl.k)), dtype=torch.uint8, device="cuda")
        sws = torch.empty(max(1, dsa.workspace_size(dsa.WS_SPARSE_MLA, batch, wl.k)), dtype=torch.uint8,
                          device="cuda")

        def three_step():
            dsa.indexer_scores(batch, dev["qi"], dev["qs"], dev["w"], dev["ki"], dev["ks"], scores)
            dsa.topk(batch, scores, wl.k, idx3, ws=tws)
            dsa.sparse_mla_fwd(batch, dev["q"], dev["kv"], idx3, wl.scale, out3, lse3, ws=sws)
        three_step()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            three_step()
        e1.record(stream)
        torch.cuda.synchronize()
        t3 = e0.elapsed_time(e1) / steps
        three = {"three_step_ms": round(t3, 4), "short_mode_ms": round(ms_per_step, 4),
                 "speedup": round(t3 / ms_per_step, 3)}
        say(f"[bench] indexer -> top-k -> sparse attention on the same inputs: {t3:.3f} ms/step "
            f"({three['speedup']:.2f}x the short-sequence mode's time)")

    cpu = None
    if not args.no_cpu_baseline:
        say("[bench] timing the CPU oracle on a sample of the workload ...")
        cpu = cpu_baseline(wl, args.cpu_seconds)
        cpu.update(cpu_info())
        say(f"[bench] CPU oracle: {cpu['value']:.2f} tokens/s on {cpu['cores']} threads ({cpu['cpu_model']})")

    cfg = {"workload": workload, "batch": b.B, "query_tokens": b.T, "cache_rows": b.N,
           "max_context": b.max_kv, "topk": wl.k, "indexer_heads": HI, "indexer_dim": DI,
           "heads": H, "d_qk": D, "d_v": DV, "entry": f"dsa_{entry}_fwd", "workspace_bytes": ws_bytes}
    if workload == "decode_64k":
        cfg["mean_context"] = round(float(np.mean(np.diff(b.cu_kv))), 1)
    if b.max_kv <= wl.k:
        cfg["entry"] += " (short-sequence mode: no indexer, no select)"
    line = {"metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
            "steps": steps, "warmup": warmup, "ms_per_step": round(ms_per_step, 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "fp8+bf16", "data": "synthetic", "config": cfg, "roofline": roof,
            "kernels": kernels, "timing": timing, "cpu_baseline": cpu}
    if three is not None:
        line["short_mode"] = three
    return line


if __name__ == "__main__":
    sys.exit(main())
