"""Seeded synthetic inputs for the DSA hot path (shared by tests, smoke and bench).

This module only draws random numbers and packs them into the storage formats
the path consumes (bf16 bits, FP8 E4M3FN codes with a per-token absmax scale,
batch descriptors).  It holds none of the method's arithmetic: no index
scores, no selection, no attention.  Neither the GPU library nor the oracle
imports it; both receive its arrays as inputs.

Randomness: numpy's PCG64 seeded through ``SeedSequence([seed, tensor_id,
(sequence,) block])`` so that any block of rows can be regenerated on its own
(the oracle then sees exactly the rows the GPU saw, at any size).  Rounding to
bf16 and FP8 uses torch's CPU casts (round to nearest even).
"""
from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

# tensor ids: one independent stream per input tensor
T_QI, T_KI, T_W, T_Q, T_KV, T_CTX = 1, 2, 3, 4, 5, 6

E4M3_MAX = 448.0  # largest finite OCP E4M3FN magnitude


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _block_rows(row_elems: int) -> int:
    return max(1, (1 << 20) // max(1, row_elems))


def normal_rows(seed: int, tid: int, row0: int, row1: int, row_elems: int,
                scale: float = 1.0, sub: int | None = None, out: np.ndarray | None = None) -> np.ndarray:
    """Rows [row0, row1) of a seeded N(0, scale^2) float32 matrix with
    ``row_elems`` columns.  Row r depends only on (seed, tid, sub, r)."""
    br = _block_rows(row_elems)
    n = row1 - row0
    if out is None:
        out = np.empty((n, row_elems), dtype=np.float32)
    b0, b1 = row0 // br, (row1 + br - 1) // br if n > 0 else row0 // br

    def fill(b):
        key = [seed, tid, b] if sub is None else [seed, tid, sub, b]
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(key)))
        blk = g.standard_normal((br, row_elems), dtype=np.float32)
        lo, hi = max(row0, b * br), min(row1, (b + 1) * br)
        if hi > lo:
            dst = out[lo - row0:hi - row0]
            np.multiply(blk[lo - b * br:hi - b * br], np.float32(scale), out=dst)

    if b1 - b0 <= 1:
        for b in range(b0, b1):
            fill(b)
    else:
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(fill, range(b0, b1)))
    return out


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def quant_e4m3_rows(x: np.ndarray):
    """Per-row absmax FP8 E4M3FN quantisation of x [rows, elems].

    scale = absmax / 448 in float32 (1 for an all-zero row); code =
    round-to-nearest-even E4M3FN of x / scale.  Returns (codes uint8, scale f32).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=1)
    scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    scale[amax == 0] = np.float32(1.0)
    y = x / scale[:, None]
    codes = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, scale


@dataclasses.dataclass
class Batch:
    """Ragged batch: query rows of sequence b are [cu_q[b], cu_q[b+1]); cache
    rows [cu_kv[b], cu_kv[b+1]); query cu_q[b]+i sits at position pos0[b]+i."""
    cu_q: np.ndarray   # int32 [B+1]
    cu_kv: np.ndarray  # int64 [B+1]
    pos0: np.ndarray   # int32 [B]

    @property
    def B(self):
        return int(self.pos0.shape[0])

    @property
    def T(self):
        return int(self.cu_q[-1])

    @property
    def N(self):
        return int(self.cu_kv[-1])

    @property
    def max_q(self):
        return int(np.max(self.cu_q[1:] - self.cu_q[:-1])) if self.B else 0

    @property
    def max_kv(self):
        return int(np.max(self.cu_kv[1:] - self.cu_kv[:-1])) if self.B else 0

    @staticmethod
    def prefill(n_q: int, n_kv: int, pos0: int) -> "Batch":
        return Batch(np.array([0, n_q], np.int32), np.array([0, n_kv], np.int64),
                     np.array([pos0], np.int32))

    @staticmethod
    def decode(ctx: np.ndarray) -> "Batch":
        ctx = np.asarray(ctx, dtype=np.int64)
        B = ctx.shape[0]
        cu_kv = np.zeros(B + 1, np.int64)
        cu_kv[1:] = np.cumsum(ctx)
        return Batch(np.arange(B + 1, dtype=np.int32), cu_kv, (ctx - 1).astype(np.int32))

    @staticmethod
    def ragged(n_q, n_kv, pos0) -> "Batch":
        n_q = np.asarray(n_q, np.int64)
        n_kv = np.asarray(n_kv, np.int64)
        cu_q = np.zeros(len(n_q) + 1, np.int32)
        cu_q[1:] = np.cumsum(n_q)
        cu_kv = np.zeros(len(n_kv) + 1, np.int64)
        cu_kv[1:] = np.cumsum(n_kv)
        return Batch(cu_q, cu_kv, np.asarray(pos0, np.int32))


@dataclasses.dataclass
class Inputs:
    """Host copies of every input of one DSA forward."""
    batch: Batch
    qi: np.ndarray       # [T, HI, DI] uint8 e4m3 codes (or float32 values when fp8=False)
    qi_scale: np.ndarray  # [T, HI] float32 (per-token value broadcast over heads)
    w: np.ndarray        # [T, HI] float32
    ki: np.ndarray       # [N, DI] uint8 e4m3 codes (or float32 values)
    ki_scale: np.ndarray  # [N] float32
    q: np.ndarray        # [T, H, D] uint16 bf16 bits (or float32 values)
    kv: np.ndarray       # [N, D] uint16 bf16 bits (or float32 values)
    HI: int
    DI: int
    H: int
    D: int
    Dv: int
    k: int
    scale: float
    seed: int


class Workload:
    """Row-addressable description of one forward's inputs.  Every row of every
    tensor is a pure function of (seed, tensor id, [sequence,] row), so the same
    values can be produced in full (small cases), streamed to the GPU in chunks
    (large cases), or regenerated for a few sampled rows (the oracle side).

    q_I, k_I ~ N(0,1) as FP8 E4M3FN with a per-token absmax scale (when fp8);
    w ~ N(0,1) * w_scale (default 1/sqrt(HI)); q, kv ~ N(0,1) rounded to bf16
    (float32 when fp8=False); softmax scale 1/sqrt(D) unless given.  With
    per_seq each sequence draws from its own streams (rows restart per sequence).
    """

    def __init__(self, batch: Batch, *, seed: int, HI=64, DI=128, H=128, D=576, Dv=512, k=2048,
                 scale: float | None = None, w_scale: float | None = None, fp8: bool = True,
                 per_seq: bool = False):
        self.batch, self.seed = batch, int(seed)
        self.HI, self.DI, self.H, self.D, self.Dv, self.k = HI, DI, H, D, Dv, k
        self.scale = float(1.0 / math.sqrt(D) if scale is None else scale)
        self.w_scale = float(1.0 / math.sqrt(HI) if w_scale is None else w_scale)
        self.fp8, self.per_seq = fp8, per_seq

    # -- row generation ------------------------------------------------------
    def _rows(self, tid, side, r0, r1, elems, scale):
        """Rows [r0, r1) (global numbering) of a query-side ('q') or cache-side
        ('kv') tensor."""
        out = np.empty((r1 - r0, elems), dtype=np.float32)
        if not self.per_seq:
            return normal_rows(self.seed, tid, r0, r1, elems, scale, out=out)
        cu = self.batch.cu_q if side == "q" else self.batch.cu_kv
        b = int(np.searchsorted(cu, r0, side="right") - 1)
        r = r0
        while r < r1:
            while int(cu[b + 1]) <= r:
                b += 1
            hi = min(r1, int(cu[b + 1]))
            lo = int(cu[b])
            normal_rows(self.seed, tid, r - lo, hi - lo, elems, scale, sub=b,
                        out=out[r - r0:hi - r0])
            r = hi
        return out

    def qi_rows(self, r0, r1):
        x = self._rows(T_QI, "q", r0, r1, self.HI * self.DI, 1.0)
        if not self.fp8:
            return x.reshape(-1, self.HI, self.DI), np.ones((r1 - r0, self.HI), np.float32)
        codes, sc = quant_e4m3_rows(x)  # one scale per token
        return (codes.reshape(-1, self.HI, self.DI),
                np.repeat(sc[:, None], self.HI, axis=1).astype(np.float32))

    def w_rows(self, r0, r1):
        return self._rows(T_W, "q", r0, r1, self.HI, self.w_scale)

    def q_rows(self, r0, r1):
        x = self._rows(T_Q, "q", r0, r1, self.H * self.D, 1.0)
        return (to_bf16_bits(x) if self.fp8 else x).reshape(-1, self.H, self.D)

    def ki_rows(self, r0, r1):
        x = self._rows(T_KI, "kv", r0, r1, self.DI, 1.0)
        if not self.fp8:
            return x, np.ones(r1 - r0, np.float32)
        return quant_e4m3_rows(x)

    def kv_rows(self, r0, r1):
        x = self._rows(T_KV, "kv", r0, r1, self.D, 1.0)
        return to_bf16_bits(x) if self.fp8 else x

    # -- assembled forms -----------------------------------------------------
    def host(self) -> "Inputs":
        T, N = self.batch.T, self.batch.N
        qi, qs = self.qi_rows(0, T)
        ki, ks = self.ki_rows(0, N)
        return Inputs(self.batch, qi, qs, self.w_rows(0, T), ki, ks, self.q_rows(0, T),
                      self.kv_rows(0, N), self.HI, self.DI, self.H, self.D, self.Dv, self.k,
                      self.scale, self.seed)

    def sampled_host(self, rows) -> "Inputs":
        """Full caches plus the query-side tensors of the given rows only: the
        other query rows stay zero in arrays allocated with np.zeros (pages
        never touched are never made resident), so the oracle can check a few
        rows of a large forward with its usual global row numbering."""
        T, N = self.batch.T, self.batch.N
        qi = np.zeros((T, self.HI, self.DI), np.uint8 if self.fp8 else np.float32)
        qs = np.zeros((T, self.HI), np.float32)
        w = np.zeros((T, self.HI), np.float32)
        q = np.zeros((T, self.H, self.D), np.uint16 if self.fp8 else np.float32)
        for t in sorted(set(int(r) for r in rows)):
            a, sc = self.qi_rows(t, t + 1)
            qi[t], qs[t] = a[0], sc[0]
            w[t] = self.w_rows(t, t + 1)[0]
            q[t] = self.q_rows(t, t + 1)[0]
        ki, ks = self.ki_rows(0, N)
        return Inputs(self.batch, qi, qs, w, ki, ks, q, self.kv_rows(0, N), self.HI, self.DI,
                      self.H, self.D, self.Dv, self.k, self.scale, self.seed)

    def device(self, device="cuda", chunk_elems: int = 1 << 26) -> dict:
        """All inputs as torch tensors on `device`, generated in row chunks."""
        T, N = self.batch.T, self.batch.N
        out = {
            "qi": torch.empty((T, self.HI, self.DI), dtype=torch.uint8, device=device),
            "qs": torch.empty((T, self.HI), dtype=torch.float32, device=device),
            "w": torch.empty((T, self.HI), dtype=torch.float32, device=device),
            "q": torch.empty((T, self.H, self.D), dtype=torch.int16, device=device),
            "ki": torch.empty((N, self.DI), dtype=torch.uint8, device=device),
            "ks": torch.empty((N,), dtype=torch.float32, device=device),
            "kv": torch.empty((N, self.D), dtype=torch.int16, device=device),
        }

        def put(name, r0, arr):
            a = np.ascontiguousarray(arr)
            if a.dtype == np.uint16:
                a = a.view(np.int16)
            out[name][r0:r0 + a.shape[0]].copy_(torch.from_numpy(a))

        step_q = max(1, chunk_elems // (self.H * self.D))
        for r0 in range(0, T, step_q):
            r1 = min(T, r0 + step_q)
            qi, qs = self.qi_rows(r0, r1)
            put("qi", r0, qi)
            put("qs", r0, qs)
            put("w", r0, self.w_rows(r0, r1))
            put("q", r0, self.q_rows(r0, r1))
        step_k = max(1, chunk_elems // self.D)
        for r0 in range(0, N, step_k):
            r1 = min(N, r0 + step_k)
            ki, ks = self.ki_rows(r0, r1)
            put("ki", r0, ki)
            put("ks", r0, ks)
            put("kv", r0, self.kv_rows(r0, r1))
        return out


def make_inputs(batch: Batch, *, seed: int, HI=64, DI=128, H=128, D=576, Dv=512, k=2048,
                scale: float | None = None, w_scale: float | None = None, fp8: bool = True,
                per_seq: bool = False) -> Inputs:
    """Full host arrays of Workload(...) (small cases)."""
    return Workload(batch, seed=seed, HI=HI, DI=DI, H=H, D=D, Dv=Dv, k=k, scale=scale,
                    w_scale=w_scale, fp8=fp8, per_seq=per_seq).host()


def decode_contexts(seed: int, B: int, lo: int = 16384, hi: int = 131072) -> np.ndarray:
    """Context lengths drawn uniformly from the integers lo..hi (inclusive)."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, T_CTX])))
    return g.integers(lo, hi + 1, size=B, dtype=np.int64)


# --- the workloads (sizes and distributions of the DSA configurations) -------

SEED_BASE = 0xD5A0


def tiny_prefill(k: int = 32) -> Inputs:
    """L=256 causal, 4 indexer heads of dim 32, 8 query heads over a 64-d latent
    + 16-d rope (value = 64-d latent); all fp32; w ~ N(0,1)/sqrt(4); scale 1/sqrt(80)."""
    return make_inputs(Batch.prefill(256, 256, 0), seed=SEED_BASE + 1, HI=4, DI=32, H=8,
                       D=80, Dv=64, k=k, fp8=False)


def prefill(L: int, seed: int = SEED_BASE + 2, k: int = 2048) -> Workload:
    """Batch 1, L causal tokens: FP8 indexer (64 heads x 128), 128-head MQA-mode
    MLA over 576-d bf16 latent rows (value = first 512)."""
    return Workload(Batch.prefill(L, L, 0), seed=seed, k=k)


def decode(B: int = 64, seed: int = SEED_BASE + 4, lo: int = 16384, hi: int = 131072,
           k: int = 2048) -> Workload:
    """B sequences, one new token each at the end of a context drawn from
    U{lo..hi}; per-sequence streams."""
    ctx = decode_contexts(seed, B, lo, hi)
    return Workload(Batch.decode(ctx), seed=seed, k=k, per_seq=True)


def chunked_prefill(n_new: int = 4096, ctx: int = 131072, seed: int = SEED_BASE + 5,
                    k: int = 2048) -> Workload:
    """n_new query tokens at positions ctx-n_new .. ctx-1 over a ctx-entry cache."""
    return Workload(Batch.prefill(n_new, ctx, ctx - n_new), seed=seed, k=k)
