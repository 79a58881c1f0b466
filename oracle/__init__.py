"""CPU oracle for the DeepSeek Sparse Attention hot path (test infrastructure).

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library does not use it, and it
imports nothing from the GPU library.

The arithmetic lives in ``dsa_oracle.c`` (plain C, double precision, OpenMP
over query rows); this module only builds it with gcc and marshals numpy
arrays into it.  See the header of ``dsa_oracle.c`` for the definitions
followed and the pages they come from.

Parity pins (tests/test_oracle_*.py) check every function here against
closed forms, library routines on special cases, brute force and invariants.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dsa_oracle.c")
# DSA_ORACLE_LIBRARY names another build of dsa_oracle.c (the AddressSanitizer
# build the CPU tests make); by default the in-tree library is used.
_ASAN_LIB = os.environ.get("DSA_ORACLE_LIBRARY")
_IN_TREE_LIB = os.path.join(_HERE, "libdsa_oracle.so")
_LIB = _ASAN_LIB or _IN_TREE_LIB
_lib = None

F32, BF16, E4M3 = 0, 1, 2


def build(force: bool = True) -> str:
    """Compile dsa_oracle.c into libdsa_oracle.so with gcc (-O2, OpenMP)."""
    out = _IN_TREE_LIB
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(_SRC):
        tmp = out + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall",
                        "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, out)
    return out


def build_asan(out: str) -> str:
    """Compile dsa_oracle.c with gcc's AddressSanitizer into ``out``.

    The library expects the sanitizer runtime to be loaded first
    (LD_PRELOAD of gcc's libasan) and is selected with DSA_ORACLE_LIBRARY.
    """
    subprocess.run(["gcc", "-O1", "-g", "-fsanitize=address", "-fno-omit-frame-pointer",
                    "-fopenmp", "-fPIC", "-shared", "-Wall", "-o", out, _SRC, "-lm"], check=True)
    return out


def lib():
    global _lib
    if _lib is None:
        if _ASAN_LIB:
            if not os.path.exists(_ASAN_LIB):
                raise FileNotFoundError(_ASAN_LIB)
        elif not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        p, i32, i64, dbl = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
        L.ora_e4m3_value.argtypes = [ctypes.c_uint8]
        L.ora_e4m3_value.restype = dbl
        L.ora_bf16_value.argtypes = [ctypes.c_uint16]
        L.ora_bf16_value.restype = dbl
        L.ora_e4m3_decode_all.argtypes = [p]
        L.ora_indexer.argtypes = [i32, p, p, p, p, i64, i32, i32, p, i32, p, p, p, i32, p, p, p, i64]
        L.ora_topk.argtypes = [i32, p, p, p, p, i64, p, i64, i32, p]
        L.ora_sparse_attn.argtypes = [i32, p, p, p, p, i64, i32, i32, i32, dbl, p, i32, p, i32, p, i32, p, p]
        L.ora_dense_attn.argtypes = [i32, p, p, p, p, i64, i32, i32, i32, dbl, p, i32, p, i32, p, p]
        L.ora_indexer_kl.argtypes = [i32, p, p, p, p, i64, i32, i32, dbl, p, i32, p, i32, p, i64, p, i32, p, p]
        L.ora_sparse_attn_bwd.argtypes = [i32, p, p, p, p, i64, i32, i32, i32, dbl, p, i32, p, i32, p, i32, p, i32,
                                          p, i32, p, p]
        L.ora_num_threads.restype = i32
        L.ora_e4m3_encode.argtypes = [ctypes.c_float]
        L.ora_e4m3_encode.restype = ctypes.c_uint8
        L.ora_quant_rows.argtypes = [p, i64, i64, p, p]
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _batch(cu_q, cu_kv, pos0):
    cu_q = np.ascontiguousarray(cu_q, dtype=np.int32)
    cu_kv = np.ascontiguousarray(cu_kv, dtype=np.int64)
    pos0 = np.ascontiguousarray(pos0, dtype=np.int32)
    assert cu_q.shape[0] == cu_kv.shape[0] == pos0.shape[0] + 1
    return cu_q, cu_kv, pos0, int(pos0.shape[0])


def _rows(rows, total):
    if rows is None:
        return None, int(total)
    r = np.ascontiguousarray(rows, dtype=np.int32)
    return r, int(r.shape[0])


def _vtype(a):
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.uint8:
        return E4M3
    raise TypeError("oracle inputs are float32 values, uint16 bf16 bits or uint8 e4m3 codes")


def num_threads() -> int:
    return int(lib().ora_num_threads())


def e4m3_value(code: int) -> float:
    return float(lib().ora_e4m3_value(int(code)))


def e4m3_table() -> np.ndarray:
    t = np.zeros(256, dtype=np.float64)
    lib().ora_e4m3_decode_all(_ptr(t))
    return t


def e4m3_encode(y: float) -> int:
    """Nearest E4M3FN code of the binary32 value y (ties to even, saturating)."""
    return int(lib().ora_e4m3_encode(float(y)))


def quant_rows(x: np.ndarray):
    """Per-group absmax E4M3FN quantisation of x [rows, cols] (binary32):
    returns (codes uint8 [rows, cols], scale float32 [rows])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, cols = x.shape
    codes = np.zeros((rows, cols), dtype=np.uint8)
    scale = np.zeros(rows, dtype=np.float32)
    if lib().ora_quant_rows(_ptr(x), rows, cols, _ptr(codes), _ptr(scale)) != 0:
        raise ValueError("ora_quant_rows: bad arguments")
    return codes, scale


def bf16_value(bits: int) -> float:
    return float(lib().ora_bf16_value(int(bits)))


def visible(cu_q, cu_kv, pos0):
    """Per query row: (sequence, cache offset, context length, position,
    visible keys) — the batch convention of dsa_oracle.c, for test bookkeeping."""
    cu_q, cu_kv, pos0, B = _batch(cu_q, cu_kv, pos0)
    T = int(cu_q[-1])
    seq = np.zeros(T, np.int64)
    for b in range(B):
        seq[cu_q[b]:cu_q[b + 1]] = b
    kv0 = cu_kv[seq]
    ctx = cu_kv[seq + 1] - cu_kv[seq]
    pos = pos0[seq].astype(np.int64) + (np.arange(T) - cu_q[seq])
    nvis = np.clip(np.minimum(pos + 1, ctx), 0, None)
    return seq, kv0, ctx, pos, nvis


def indexer(cu_q, cu_kv, pos0, q, q_scale, w, k, k_scale, rows=None, ld=None, want_abs=False):
    """Index scores I[t, s] (float32, -inf where masked) for the given rows.

    q: [T, HI, DI] float32 values or uint8 e4m3 codes (then q_scale [T, HI]).
    k: [N, DI]     float32 values or uint8 e4m3 codes (then k_scale [N]).
    w: [T, HI] float32.  Returns scores [nrows, ld] and, if want_abs, the
    absolute-term sums A [nrows, ld] (float64).  Columns at or beyond the
    sequence's context length are left as NaN.
    """
    cu_q, cu_kv, pos0, B = _batch(cu_q, cu_kv, pos0)
    T, HI, DI = q.shape
    r, nrows = _rows(rows, T)
    if ld is None:
        ld = int(np.max(cu_kv[1:] - cu_kv[:-1])) if B else 0
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    w = np.ascontiguousarray(w, dtype=np.float32)
    qs = None if q_scale is None else np.ascontiguousarray(q_scale, dtype=np.float32)
    ks = None if k_scale is None else np.ascontiguousarray(k_scale, dtype=np.float32)
    scores = np.full((nrows, ld), np.nan, dtype=np.float32)
    absum = np.full((nrows, ld), np.nan, dtype=np.float64) if want_abs else None
    rc = lib().ora_indexer(B, _ptr(cu_q), _ptr(cu_kv), _ptr(pos0), _ptr(r), nrows, HI, DI,
                           _ptr(q), _vtype(q), _ptr(qs), _ptr(w), _ptr(k), _vtype(k), _ptr(ks),
                           _ptr(scores), _ptr(absum), ld)
    if rc != 0:
        raise ValueError("ora_indexer failed (bad batch description or allocation)")
    return (scores, absum) if want_abs else scores


def topk(cu_q, cu_kv, pos0, scores, k, rows=None):
    """Top-k positions per row from oracle scores [nrows, ld]: ascending, -1 padded."""
    cu_q, cu_kv, pos0, B = _batch(cu_q, cu_kv, pos0)
    r, nrows = _rows(rows, int(cu_q[-1]))
    assert scores.shape[0] == nrows
    scores = np.ascontiguousarray(scores, dtype=np.float32)
    idx = np.empty((nrows, k), dtype=np.int32)
    rc = lib().ora_topk(B, _ptr(cu_q), _ptr(cu_kv), _ptr(pos0), _ptr(r), nrows,
                        _ptr(scores), scores.shape[1], k, _ptr(idx))
    if rc != 0:
        raise ValueError("ora_topk failed")
    return idx


def sparse_attn(cu_q, cu_kv, pos0, q, kv, idx, Dv, scale, rows=None):
    """MQA-mode attention over idx rows. q [T,H,D], kv [N,D] float32 or bf16
    bits (uint16); idx [nrows, k]. Returns o [nrows,H,Dv] f32, lse [nrows,H] f32."""
    cu_q, cu_kv, pos0, B = _batch(cu_q, cu_kv, pos0)
    T, H, D = q.shape
    r, nrows = _rows(rows, T)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    assert idx.shape[0] == nrows
    q = np.ascontiguousarray(q)
    kv = np.ascontiguousarray(kv)
    o = np.empty((nrows, H, Dv), dtype=np.float32)
    lse = np.empty((nrows, H), dtype=np.float32)
    rc = lib().ora_sparse_attn(B, _ptr(cu_q), _ptr(cu_kv), _ptr(pos0), _ptr(r), nrows, H, D, Dv,
                               float(scale), _ptr(q), _vtype(q), _ptr(kv), _vtype(kv),
                               _ptr(idx), idx.shape[1], _ptr(o), _ptr(lse))
    if rc != 0:
        raise ValueError("ora_sparse_attn failed (index out of range or bad batch)")
    return o, lse


def dense_attn(cu_q, cu_kv, pos0, q, kv, Dv, scale, rows=None):
    """Brute-force causal MQA attention over every visible key."""
    cu_q, cu_kv, pos0, B = _batch(cu_q, cu_kv, pos0)
    T, H, D = q.shape
    r, nrows = _rows(rows, T)
    q = np.ascontiguousarray(q)
    kv = np.ascontiguousarray(kv)
    o = np.empty((nrows, H, Dv), dtype=np.float32)
    lse = np.empty((nrows, H), dtype=np.float32)
    rc = lib().ora_dense_attn(B, _ptr(cu_q), _ptr(cu_kv), _ptr(pos0), _ptr(r), nrows, H, D, Dv,
                              float(scale), _ptr(q), _vtype(q), _ptr(kv), _vtype(kv),
                              _ptr(o), _ptr(lse))
    if rc != 0:
        raise ValueError("ora_dense_attn failed")
    return o, lse


def indexer_kl(cu_q, cu_kv, pos0, q, kv, scale, scores, idx=None, rows=None, want_p=False):
    """Indexer KL loss per row (the target: head-summed, L1-normalised main
    attention over the key set; the loss: KL(target || softmax of the index
    scores) over the same set).  idx None: dense warm-up over every visible
    key; else the sparse stage over the slots idx [nrows, k].  scores
    [nrows, ld] f32 hold I at column s.  Returns kl [nrows] f64 and, if
    want_p, the target p ([nrows, k] per slot, or [nrows, ld] per column with
    NaN beyond the visible keys)."""
    cu_q, cu_kv, pos0, B = _batch(cu_q, cu_kv, pos0)
    T, H, D = q.shape
    r, nrows = _rows(rows, T)
    scores = np.ascontiguousarray(scores, dtype=np.float32)
    assert scores.shape[0] == nrows
    ld = scores.shape[1]
    q = np.ascontiguousarray(q)
    kv = np.ascontiguousarray(kv)
    k = 0
    if idx is not None:
        idx = np.ascontiguousarray(idx, dtype=np.int32)
        assert idx.shape[0] == nrows
        k = idx.shape[1]
    kl = np.empty(nrows, dtype=np.float64)
    p = None
    if want_p:
        p = np.full((nrows, k if idx is not None else ld), np.nan, dtype=np.float64)
    rc = lib().ora_indexer_kl(B, _ptr(cu_q), _ptr(cu_kv), _ptr(pos0), _ptr(r), nrows, H, D, float(scale),
                              _ptr(q), _vtype(q), _ptr(kv), _vtype(kv), _ptr(scores), ld,
                              _ptr(idx), k, _ptr(kl), _ptr(p))
    if rc != 0:
        raise ValueError("ora_indexer_kl failed (index out of range or bad batch)")
    return (kl, p) if want_p else kl


def sparse_attn_bwd(cu_q, cu_kv, pos0, q, kv, dout, idx, Dv, scale, rows=None, out=None):
    """Backward of the sparse MQA attention over idx rows [nrows, k]: given
    dout = dL/do [T, H, Dv] (float32 or bf16 bits), returns dq [nrows, H, D]
    and dkv [N, D] (float64; dkv holds the contributions of the rows asked for).
    out [T, H, Dv] (optional): the forward output delta = <dout, out> is taken
    from (as a backward handed the forward's rounded output does); default:
    the exact output."""
    cu_q, cu_kv, pos0, B = _batch(cu_q, cu_kv, pos0)
    T, H, D = q.shape
    N = kv.shape[0]
    r, nrows = _rows(rows, T)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    assert idx.shape[0] == nrows
    q = np.ascontiguousarray(q)
    kv = np.ascontiguousarray(kv)
    dout = np.ascontiguousarray(dout)
    assert dout.shape == (T, H, Dv)
    if out is not None:
        out = np.ascontiguousarray(out)
        assert out.shape == (T, H, Dv)
    dq = np.empty((nrows, H, D), dtype=np.float64)
    dkv = np.zeros((N, D), dtype=np.float64)
    rc = lib().ora_sparse_attn_bwd(B, _ptr(cu_q), _ptr(cu_kv), _ptr(pos0), _ptr(r), nrows, H, D, Dv, float(scale),
                                   _ptr(q), _vtype(q), _ptr(kv), _vtype(kv), _ptr(dout), _vtype(dout),
                                   _ptr(out), _vtype(out) if out is not None else 0,
                                   _ptr(idx), idx.shape[1], _ptr(dq), _ptr(dkv))
    if rc != 0:
        raise ValueError("ora_sparse_attn_bwd failed (index out of range or bad batch)")
    return dq, dkv
