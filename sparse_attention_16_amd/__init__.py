"""MI355X (gfx950) DeepSeek Sparse Attention hot path: Python binding.

Thin ctypes layer over ``libdsa.so`` (the C ABI declared in ``include/dsa.h``):
it marshals torch device tensors into pointers and calls the library; every
step of the path runs in the library's HIP kernels.  PyTorch provides device
memory and streams only.  Importing this package fails loudly when the built
library is missing: there is no fallback implementation.

Entry points (same names as the C ABI, without the ``dsa_`` prefix):
    indexer_scores, indexer_topk, topk, sparse_mla_fwd, dense_mla_fwd, indexer_kl_fwd, sparse_mla_bwd, prefill_fwd,
    decode_fwd, fwd_profile (measurement helper), check_selection (validation),
    quantize_queries, append_cache,
    workspace_size, status_string, version
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# DSA_LIBRARY names another build of the same library (the host-sanitised
# build the CPU tests make); by default the in-tree libdsa.so is loaded.
LIB_PATH = os.environ.get("DSA_LIBRARY") or os.path.join(_PKG, "libdsa.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python -m sparse_attention_16_amd.build` "
        "(hipcc, gfx950) before importing sparse_attention_16_amd")

_lib = ctypes.CDLL(LIB_PATH)

DSA_OK, DSA_ERR_INVALID_ARG, DSA_ERR_UNSUPPORTED, DSA_ERR_WORKSPACE, DSA_ERR_HIP, DSA_ERR_CHECK = range(6)
(WS_TOPK, WS_SPARSE_MLA, WS_PREFILL, WS_DECODE, WS_DENSE_MLA, WS_INDEXER_KL, WS_SPARSE_MLA_BWD,
 WS_INDEXER_TOPK) = range(8)

EXPORTS = ("dsa_indexer_scores", "dsa_indexer_topk", "dsa_topk", "dsa_sparse_mla_fwd", "dsa_dense_mla_fwd", "dsa_indexer_kl_fwd",
           "dsa_sparse_mla_bwd", "dsa_prefill_fwd",
           "dsa_decode_fwd", "dsa_decode_fwd_noalloc", "dsa_decode_fwd_noalloc_max_bytes", "dsa_fwd_profile",
           "dsa_check_selection", "dsa_measure_peaks", "dsa_quantize_queries", "dsa_append_cache",
           "dsa_workspace_size",
           "dsa_status_string", "dsa_version")


class DsaError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} (status {status})")
        self.status = status


class dsa_batch(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("total_q", ctypes.c_int32),
                ("max_q", ctypes.c_int32), ("max_kv", ctypes.c_int32),
                ("total_kv", ctypes.c_int64), ("cu_q", ctypes.c_void_p),
                ("cu_kv", ctypes.c_void_p), ("pos0", ctypes.c_void_p)]


class dsa_fwd_args(ctypes.Structure):
    _fields_ = [("batch", dsa_batch), ("q_fp8", ctypes.c_void_p), ("q_scale", ctypes.c_void_p),
                ("w", ctypes.c_void_p), ("k_fp8", ctypes.c_void_p), ("k_scale", ctypes.c_void_p),
                ("q", ctypes.c_void_p), ("kv", ctypes.c_void_p),
                ("HI", ctypes.c_int32), ("DI", ctypes.c_int32), ("H", ctypes.c_int32),
                ("D", ctypes.c_int32), ("Dv", ctypes.c_int32), ("k", ctypes.c_int32),
                ("scale", ctypes.c_float)]


class dsa_kernel_time(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_char_p), ("ms", ctypes.c_float), ("items", ctypes.c_int64)]


class dsa_peaks(ctypes.Structure):
    _fields_ = [("bf16_tflops", ctypes.c_double), ("fp8_tflops", ctypes.c_double),
                ("hbm_read_gbs", ctypes.c_double), ("hbm_copy_gbs", ctypes.c_double)]


_P, _I, _I64, _SZ, _F = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
_BP = ctypes.POINTER(dsa_batch)
_lib.dsa_indexer_scores.argtypes = [_BP, _P, _P, _P, _P, _P, _I, _I, _P, _I64, _P]
_lib.dsa_topk.argtypes = [_BP, _P, _I64, _I, _P, _P, _SZ, _P]
_lib.dsa_indexer_topk.argtypes = [_BP, _P, _P, _P, _P, _P, _I, _I, _I, _P, _P, _SZ, _P]
_lib.dsa_sparse_mla_fwd.argtypes = [_BP, _P, _P, _P, _I, _I, _I, _I, _F, _P, _P, _P, _SZ, _P]
_lib.dsa_dense_mla_fwd.argtypes = [_BP, _P, _P, _I, _I, _I, _F, _P, _P, _P, _SZ, _P]
_lib.dsa_indexer_kl_fwd.argtypes = [_BP, _P, _P, _P, _I, _I, _F, _P, _I64, _P, _I, _P, _P, _P, _SZ, _P]
_lib.dsa_sparse_mla_bwd.argtypes = [_BP, _P, _P, _P, _I, _I, _I, _I, _F, _P, _P, _P, _P, _P, _P, _SZ, _P]
_lib.dsa_prefill_fwd.argtypes = [ctypes.POINTER(dsa_fwd_args), _P, _P, _P, _P, _SZ, _P]
_lib.dsa_decode_fwd.argtypes = [ctypes.POINTER(dsa_fwd_args), _P, _P, _P, _P, _SZ, _P]
_lib.dsa_decode_fwd_noalloc.argtypes = [ctypes.POINTER(dsa_fwd_args), _P, _P, _P, _P]
_lib.dsa_decode_fwd_noalloc_max_bytes.restype = _SZ
_lib.dsa_fwd_profile.argtypes = [ctypes.POINTER(dsa_fwd_args), _I, _P, _P, _P, _P, _SZ, _P,
                                 ctypes.POINTER(dsa_kernel_time), _I, ctypes.POINTER(ctypes.c_int)]
_lib.dsa_check_selection.argtypes = [_BP, _P, _I, _P, ctypes.POINTER(ctypes.c_int)]
_lib.dsa_measure_peaks.argtypes = [_P, _SZ, _P, ctypes.POINTER(dsa_peaks)]
_lib.dsa_workspace_size.argtypes = [_I, _BP, _I, _I, _I]
_lib.dsa_quantize_queries.argtypes = [_P, _I64, _I, _I, _P, _P, _P]
_lib.dsa_append_cache.argtypes = [_P, _P, _I64, _I, _I, _P, _P, _P, _P, _I64, _P]
_lib.dsa_workspace_size.restype = _SZ
_lib.dsa_status_string.argtypes = [_I]
_lib.dsa_status_string.restype = ctypes.c_char_p
_lib.dsa_version.restype = ctypes.c_char_p
for _name in ("dsa_indexer_scores", "dsa_indexer_topk", "dsa_topk", "dsa_sparse_mla_fwd", "dsa_prefill_fwd",
              "dsa_decode_fwd", "dsa_decode_fwd_noalloc", "dsa_fwd_profile"):
    getattr(_lib, _name).restype = ctypes.c_int


def status_string(status: int) -> str:
    return _lib.dsa_status_string(int(status)).decode()


def version() -> str:
    return _lib.dsa_version().decode()


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check(status: int, what: str):
    if status != DSA_OK:
        raise DsaError(status, what)


class Batch:
    """Device-side ragged batch descriptor (cu_q, cu_kv, pos0 on the GPU) plus
    the host scalars the C ABI wants.  Build from host arrays with
    ``Batch.from_host(cu_q, cu_kv, pos0, device)``."""

    def __init__(self, cu_q, cu_kv, pos0, total_q, max_q, total_kv, max_kv):
        self.cu_q, self.cu_kv, self.pos0 = cu_q, cu_kv, pos0
        self.B = int(pos0.numel())
        self.total_q, self.max_q = int(total_q), int(max_q)
        self.total_kv, self.max_kv = int(total_kv), int(max_kv)
        self.c = dsa_batch(self.B, self.total_q, self.max_q, self.max_kv, self.total_kv,
                           _ptr(cu_q), _ptr(cu_kv), _ptr(pos0))

    @staticmethod
    def from_host(cu_q, cu_kv, pos0, device="cuda"):
        import numpy as np
        cu_q = np.asarray(cu_q, np.int32)
        cu_kv = np.asarray(cu_kv, np.int64)
        pos0 = np.asarray(pos0, np.int32)
        nq = cu_q[1:] - cu_q[:-1]
        nkv = cu_kv[1:] - cu_kv[:-1]
        return Batch(torch.from_numpy(cu_q).to(device), torch.from_numpy(cu_kv).to(device),
                     torch.from_numpy(pos0).to(device), cu_q[-1], nq.max() if len(nq) else 0,
                     cu_kv[-1], nkv.max() if len(nkv) else 0)


def workspace_size(entry: int, batch: Batch, k: int, H: int = 128, Dv: int = 512) -> int:
    return int(_lib.dsa_workspace_size(int(entry), ctypes.byref(batch.c), int(k), int(H), int(Dv)))


def _workspace(entry, batch, k, ws, device):
    need = workspace_size(entry, batch, k)
    if ws is None and need > 0:
        ws = torch.empty(need, dtype=torch.uint8, device=device)
    return ws, (ws.numel() * ws.element_size() if ws is not None else 0)


def indexer_scores(batch: Batch, q_fp8, q_scale, w, k_fp8, k_scale, scores, ld=None, stream=None):
    """Index scores into ``scores`` [T, ld] fp32 (see dsa_indexer_scores)."""
    ld = scores.shape[1] if ld is None else ld
    st = _lib.dsa_indexer_scores(ctypes.byref(batch.c), _ptr(q_fp8), _ptr(q_scale), _ptr(w),
                                 _ptr(k_fp8), _ptr(k_scale), q_fp8.shape[1], q_fp8.shape[2],
                                 _ptr(scores), int(ld), _stream(stream))
    _check(st, "dsa_indexer_scores")
    return scores


def indexer_topk(batch: Batch, q_fp8, q_scale, w, k_fp8, k_scale, k: int, idx, ws=None, stream=None):
    """Top-k positions per row into ``idx`` [T, k] int32 straight from the
    indexer inputs, without a score matrix (see dsa_indexer_topk)."""
    ws, nbytes = _workspace(WS_INDEXER_TOPK, batch, k, ws, q_fp8.device)
    st = _lib.dsa_indexer_topk(ctypes.byref(batch.c), _ptr(q_fp8), _ptr(q_scale), _ptr(w), _ptr(k_fp8),
                               _ptr(k_scale), q_fp8.shape[1], q_fp8.shape[2], int(k), _ptr(idx), _ptr(ws), nbytes,
                               _stream(stream))
    _check(st, "dsa_indexer_topk")
    return idx


def quantize_queries(q, q_fp8, q_scale, stream=None):
    """FP8 E4M3FN quantisation of indexer queries q [T, 64, 128] fp32 into
    q_fp8 [T, 64, 128] uint8 and q_scale [T, 64] fp32 (see dsa_quantize_queries)."""
    st = _lib.dsa_quantize_queries(_ptr(q), q.shape[0], q.shape[1], q.shape[2], _ptr(q_fp8), _ptr(q_scale),
                                   _stream(stream))
    _check(st, "dsa_quantize_queries")
    return q_fp8, q_scale


def append_cache(k_new, kv_new, dst_rows, k_fp8, k_scale, kv, stream=None):
    """Quantise new indexer keys k_new [R, 128] fp32 into rows dst_rows of the
    FP8 key cache (k_fp8 [N, 128] uint8, k_scale [N] fp32) and copy the new
    latent rows kv_new [R, 576] bf16 (or None) into kv [N, 576] (see
    dsa_append_cache)."""
    D = kv.shape[1] if kv is not None else 576
    st = _lib.dsa_append_cache(_ptr(k_new), _ptr(kv_new), k_new.shape[0], k_new.shape[1], D, _ptr(dst_rows),
                               _ptr(k_fp8), _ptr(k_scale), _ptr(kv), k_fp8.shape[0], _stream(stream))
    _check(st, "dsa_append_cache")


def topk(batch: Batch, scores, k: int, idx, ld=None, ws=None, stream=None):
    """Top-k columns per row into ``idx`` [T, k] int32 (see dsa_topk)."""
    ld = scores.shape[1] if ld is None else ld
    ws, nbytes = _workspace(WS_TOPK, batch, k, ws, scores.device)
    st = _lib.dsa_topk(ctypes.byref(batch.c), _ptr(scores), int(ld), int(k), _ptr(idx), _ptr(ws),
                       nbytes, _stream(stream))
    _check(st, "dsa_topk")
    return idx


def sparse_mla_fwd(batch: Batch, q, kv, idx, scale: float, out, lse, Dv: int = 512, ws=None,
                   stream=None):
    """Sparse MQA-mode attention over idx rows (see dsa_sparse_mla_fwd)."""
    k = idx.shape[1]
    ws, nbytes = _workspace(WS_SPARSE_MLA, batch, k, ws, q.device)
    st = _lib.dsa_sparse_mla_fwd(ctypes.byref(batch.c), _ptr(q), _ptr(kv), _ptr(idx), int(k),
                                 q.shape[1], q.shape[2], int(Dv), float(scale), _ptr(out), _ptr(lse),
                                 _ptr(ws), nbytes, _stream(stream))
    _check(st, "dsa_sparse_mla_fwd")
    return out, lse


def dense_mla_fwd(batch: Batch, q, kv, scale: float, out, lse, Dv: int = 512, ws=None, stream=None):
    """Dense masked attention of every row over all its visible keys, the
    short-sequence mode (see dsa_dense_mla_fwd)."""
    ws, nbytes = _workspace(WS_DENSE_MLA, batch, 1, ws, q.device)
    st = _lib.dsa_dense_mla_fwd(ctypes.byref(batch.c), _ptr(q), _ptr(kv), q.shape[1], q.shape[2], int(Dv),
                                float(scale), _ptr(out), _ptr(lse), _ptr(ws), nbytes, _stream(stream))
    _check(st, "dsa_dense_mla_fwd")
    return out, lse


def indexer_kl_fwd(batch: Batch, q, kv, lse, scale: float, scores, kl, idx=None, p_out=None, ld=None, ws=None,
                   stream=None):
    """Indexer KL loss per row into kl [T] (see dsa_indexer_kl_fwd); idx None
    is the dense warm-up over every visible key."""
    ld = scores.shape[1] if ld is None else ld
    k = idx.shape[1] if idx is not None else 1
    ws, nbytes = _workspace(WS_INDEXER_KL, batch, k, ws, q.device)
    st = _lib.dsa_indexer_kl_fwd(ctypes.byref(batch.c), _ptr(q), _ptr(kv), _ptr(lse), q.shape[1], q.shape[2],
                                 float(scale), _ptr(scores), int(ld), _ptr(idx), int(k), _ptr(kl), _ptr(p_out),
                                 _ptr(ws), nbytes, _stream(stream))
    _check(st, "dsa_indexer_kl_fwd")
    return kl


def sparse_mla_bwd(batch: Batch, q, kv, idx, scale: float, out, lse, dout, dq, dkv, Dv: int = 512, ws=None,
                   stream=None):
    """Backward of sparse_mla_fwd over the same idx: dq [T, H, D] fp32 and
    dkv [N, D] fp32 (overwritten) from dout [T, H, Dv] bf16 and the forward's
    out and lse (see dsa_sparse_mla_bwd)."""
    k = idx.shape[1]
    ws, nbytes = _workspace(WS_SPARSE_MLA_BWD, batch, k, ws, q.device)
    st = _lib.dsa_sparse_mla_bwd(ctypes.byref(batch.c), _ptr(q), _ptr(kv), _ptr(idx), int(k), q.shape[1],
                                 q.shape[2], int(Dv), float(scale), _ptr(out), _ptr(lse), _ptr(dout), _ptr(dq),
                                 _ptr(dkv), _ptr(ws), nbytes, _stream(stream))
    _check(st, "dsa_sparse_mla_bwd")
    return dq, dkv


def fwd_args(batch: Batch, q_fp8, q_scale, w, k_fp8, k_scale, q, kv, k: int, scale: float,
             Dv: int = 512) -> dsa_fwd_args:
    return dsa_fwd_args(batch.c, _ptr(q_fp8), _ptr(q_scale), _ptr(w), _ptr(k_fp8), _ptr(k_scale),
                        _ptr(q), _ptr(kv), q_fp8.shape[1], q_fp8.shape[2], q.shape[1], q.shape[2],
                        int(Dv), int(k), float(scale))


def _fwd(fn, entry, what, args: dsa_fwd_args, batch: Batch, out, lse, idx_out, ws, stream):
    ws, nbytes = _workspace(entry, batch, args.k, ws, out.device)
    st = fn(ctypes.byref(args), _ptr(out), _ptr(lse), _ptr(idx_out), _ptr(ws), nbytes,
            _stream(stream))
    _check(st, what)
    return out, lse


def prefill_fwd(args: dsa_fwd_args, batch: Batch, out, lse, idx_out=None, ws=None, stream=None):
    """Whole hot path (indexer -> top-k -> sparse MLA), prefill-tuned."""
    return _fwd(_lib.dsa_prefill_fwd, WS_PREFILL, "dsa_prefill_fwd", args, batch, out, lse,
                idx_out, ws, stream)


def decode_fwd(args: dsa_fwd_args, batch: Batch, out, lse, idx_out=None, ws=None, stream=None):
    """Whole hot path (indexer -> top-k -> sparse MLA), decode-tuned (split-KV)."""
    return _fwd(_lib.dsa_decode_fwd, WS_DECODE, "dsa_decode_fwd", args, batch, out, lse,
                idx_out, ws, stream)


def decode_fwd_noalloc(args: dsa_fwd_args, out, lse, idx_out=None, stream=None):
    """dsa_decode_fwd on the library's static scratch (no workspace, no
    allocation; see dsa_decode_fwd_noalloc)."""
    st = _lib.dsa_decode_fwd_noalloc(ctypes.byref(args), _ptr(out), _ptr(lse), _ptr(idx_out), _stream(stream))
    _check(st, "dsa_decode_fwd_noalloc")
    return out, lse


def fwd_profile(args: dsa_fwd_args, batch: Batch, out, lse, idx_out=None, ws=None, decode=False, stream=None):
    """Runs the prefill (or decode) entry with a HIP event after each launch,
    waits for it, and returns [(kernel name, ms, items)] in launch order (see
    dsa_fwd_profile; items: candidates for the fused select, recomputed rows
    for the recompute, else -1)."""
    entry = WS_DECODE if decode else WS_PREFILL
    ws, nbytes = _workspace(entry, batch, args.k, ws, out.device)
    times = (dsa_kernel_time * 16)()
    n = ctypes.c_int(0)
    st = _lib.dsa_fwd_profile(ctypes.byref(args), int(bool(decode)), _ptr(out), _ptr(lse), _ptr(idx_out), _ptr(ws),
                              nbytes, _stream(stream), times, 16, ctypes.byref(n))
    _check(st, "dsa_fwd_profile")
    return [(times[i].kernel.decode(), float(times[i].ms), int(times[i].items)) for i in range(n.value)]


def check_selection(batch: Batch, idx, k: int = None, stream=None) -> int:
    """Rows of idx [T, k] that break the top-k selection contract (see
    dsa_check_selection; waits for the stream)."""
    k = idx.shape[1] if k is None else k
    bad = ctypes.c_int(-1)
    st = _lib.dsa_check_selection(ctypes.byref(batch.c), _ptr(idx), int(k), _stream(stream), ctypes.byref(bad))
    _check(st, "dsa_check_selection")
    return bad.value


def measure_peaks(buf, stream=None) -> dict:
    """Attainable bf16 / FP8 MFMA TFLOP/s and HBM read / copy GB/s on this
    GPU (see dsa_measure_peaks; `buf` is a device scratch tensor of at least
    64 MiB whose contents are overwritten; waits for the stream)."""
    r = dsa_peaks()
    st = _lib.dsa_measure_peaks(_ptr(buf), buf.numel() * buf.element_size(), _stream(stream), ctypes.byref(r))
    _check(st, "dsa_measure_peaks")
    return {"bf16_tflops": r.bf16_tflops, "fp8_tflops": r.fp8_tflops, "hbm_read_gbs": r.hbm_read_gbs,
            "hbm_copy_gbs": r.hbm_copy_gbs}


def raw_lib():
    """The loaded ctypes library (for symbol checks and direct C-ABI calls)."""
    return _lib
