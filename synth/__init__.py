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


def _seq_rows(batch: Batch, seed, tid, which: str, elems: int, scale: float, per_seq: bool):
    """Generate query-side (which='q') or cache-side (which='kv') rows; with
    per_seq each sequence has its own stream (rows restart at 0 per sequence)."""
    cu = batch.cu_q if which == "q" else batch.cu_kv
    total = int(cu[-1])
    out = np.empty((total, elems), dtype=np.float32)
    if not per_seq:
        normal_rows(seed, tid, 0, total, elems, scale, out=out)
        return out
    for b in range(batch.B):
        lo, hi = int(cu[b]), int(cu[b + 1])
        if hi > lo:
            normal_rows(seed, tid, 0, hi - lo, elems, scale, sub=b, out=out[lo:hi])
    return out


def make_inputs(batch: Batch, *, seed: int, HI=64, DI=128, H=128, D=576, Dv=512, k=2048,
                scale: float | None = None, w_scale: float | None = None, fp8: bool = True,
                per_seq: bool = False) -> Inputs:
    """Inputs for one forward: q_I, k_I ~ N(0,1) (FP8 E4M3FN with per-token
    absmax scale when fp8), w ~ N(0,1)*w_scale (default 1/sqrt(HI), i.e. 1/8 at
    64 heads), q and kv ~ N(0,1) rounded to bf16 (float32 when fp8=False),
    softmax scale 1/sqrt(D) unless given."""
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if w_scale is None:
        w_scale = 1.0 / math.sqrt(HI)
    T, N = batch.T, batch.N
    qi = _seq_rows(batch, seed, T_QI, "q", HI * DI, 1.0, per_seq)
    ki = _seq_rows(batch, seed, T_KI, "kv", DI, 1.0, per_seq)
    w = _seq_rows(batch, seed, T_W, "q", HI, w_scale, per_seq)
    q = _seq_rows(batch, seed, T_Q, "q", H * D, 1.0, per_seq)
    kv = _seq_rows(batch, seed, T_KV, "kv", D, 1.0, per_seq)
    if fp8:
        qi_codes, qs = quant_e4m3_rows(qi)          # one scale per token
        qi = qi_codes.reshape(T, HI, DI)
        qi_scale = np.repeat(qs[:, None], HI, axis=1).astype(np.float32)
        ki, ki_scale = quant_e4m3_rows(ki)
        q = to_bf16_bits(q).reshape(T, H, D)
        kv = to_bf16_bits(kv)
    else:
        qi = qi.reshape(T, HI, DI)
        qi_scale = np.ones((T, HI), np.float32)
        ki_scale = np.ones(N, np.float32)
        q = q.reshape(T, H, D)
    return Inputs(batch, qi, qi_scale, w.reshape(T, HI), ki, ki_scale, q, kv,
                  HI, DI, H, D, Dv, k, float(scale), seed)


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


def prefill(L: int, seed: int = SEED_BASE + 2, k: int = 2048) -> Inputs:
    """Batch 1, L causal tokens: FP8 indexer (64 heads x 128), 128-head MQA-mode
    MLA over 576-d bf16 latent rows (value = first 512)."""
    return make_inputs(Batch.prefill(L, L, 0), seed=seed, k=k)


def decode(B: int = 64, seed: int = SEED_BASE + 4, lo: int = 16384, hi: int = 131072,
           k: int = 2048) -> Inputs:
    """B sequences, one new token each at the end of a context drawn from
    U{lo..hi}; per-sequence streams."""
    ctx = decode_contexts(seed, B, lo, hi)
    return make_inputs(Batch.decode(ctx), seed=seed, k=k, per_seq=True)


def chunked_prefill(n_new: int = 4096, ctx: int = 131072, seed: int = SEED_BASE + 5,
                    k: int = 2048) -> Inputs:
    """n_new query tokens at positions ctx-n_new .. ctx-1 over a ctx-entry cache."""
    return make_inputs(Batch.prefill(n_new, ctx, ctx - n_new), seed=seed, k=k)
