"""Host-side checks of the C ABI (include/dsa.h): the library loads, exports
every declared entry point, sizes workspaces, and rejects bad arguments with
the documented status before launching anything.  No GPU is touched: every
call here returns from host validation (fake, aligned pointer values are never
dereferenced)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.environ.get("DSA_LIBRARY") or os.path.join(ROOT, "sparse_attention_16_amd", "libdsa.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libdsa.so not built")


@pytest.fixture(scope="module")
def dsa():
    import sparse_attention_16_amd as m
    return m


def _declared_symbols():
    text = open(os.path.join(ROOT, "include", "dsa.h")).read()
    return sorted(set(re.findall(r"\b(dsa_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(dsa):
    syms = _declared_symbols()
    assert set(syms) == set(dsa.EXPORTS)
    lib = dsa.raw_lib()
    for s in syms:
        assert hasattr(lib, s), s


def test_status_strings_and_version(dsa):
    assert dsa.status_string(0) == "ok"
    assert "unsupported" in dsa.status_string(2)
    assert "workspace" in dsa.status_string(3)
    assert "debug check" in dsa.status_string(5)
    assert "gfx950" in dsa.version()


FAKE = 1 << 20  # aligned, never dereferenced


def _batch(dsa, T=4096, N=4096, B=1, max_q=None, max_kv=None):
    return dsa.dsa_batch(B, T, T if max_q is None else max_q, N if max_kv is None else max_kv, N,
                         FAKE, FAKE, FAKE)


def test_workspace_sizes(dsa):
    lib = dsa.raw_lib()
    b = _batch(dsa, 4096, 4096)
    # one chunk of top-k: no workspace; 4096 rows: no split-KV
    assert lib.dsa_workspace_size(dsa.WS_TOPK, ctypes.byref(b), 2048, 128, 512) == 0
    assert lib.dsa_workspace_size(dsa.WS_SPARSE_MLA, ctypes.byref(b), 2048, 128, 512) == 0
    pre = lib.dsa_workspace_size(dsa.WS_PREFILL, ctypes.byref(b), 2048, 128, 512)
    assert pre >= 4096 * 4096 * 4 + 4096 * 2048 * 4
    # decode-like: 64 rows over 131072-long rows -> chunked top-k and split-KV
    d = _batch(dsa, 64, 64 * 131072, B=64, max_q=1, max_kv=131072)
    assert lib.dsa_workspace_size(dsa.WS_TOPK, ctypes.byref(d), 2048, 128, 512) >= 64 * 4 * 2048 * 8
    assert lib.dsa_workspace_size(dsa.WS_SPARSE_MLA, ctypes.byref(d), 2048, 128, 512) > 0
    # invalid arguments -> 0
    assert lib.dsa_workspace_size(dsa.WS_PREFILL, ctypes.byref(b), 0, 128, 512) == 0
    assert lib.dsa_workspace_size(dsa.WS_PREFILL, ctypes.byref(b), 2048, 64, 512) == 0
    assert lib.dsa_workspace_size(dsa.WS_PREFILL, None, 2048, 128, 512) == 0


def test_indexer_validation(dsa):
    lib = dsa.raw_lib()
    b = _batch(dsa)
    args = [FAKE] * 5
    assert lib.dsa_indexer_scores(None, *args, 64, 128, FAKE, 4096, None) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_indexer_scores(ctypes.byref(b), *args, 32, 128, FAKE, 4096, None) == dsa.DSA_ERR_UNSUPPORTED
    assert lib.dsa_indexer_scores(ctypes.byref(b), *args, 64, 64, FAKE, 4096, None) == dsa.DSA_ERR_UNSUPPORTED
    assert lib.dsa_indexer_scores(ctypes.byref(b), None, *args[1:], 64, 128, FAKE, 4096, None) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_indexer_scores(ctypes.byref(b), *args, 64, 128, FAKE, 4095, None) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_indexer_scores(ctypes.byref(b), FAKE + 4, *args[1:], 64, 128, FAKE, 4096, None) == dsa.DSA_ERR_INVALID_ARG
    bad = _batch(dsa, B=0)
    assert lib.dsa_indexer_scores(ctypes.byref(bad), *args, 64, 128, FAKE, 4096, None) == dsa.DSA_ERR_INVALID_ARG
    bad = dsa.dsa_batch(1, 10, 10, 10, 10, None, FAKE, FAKE)
    assert lib.dsa_indexer_scores(ctypes.byref(bad), *args, 64, 128, FAKE, 4096, None) == dsa.DSA_ERR_INVALID_ARG
    empty = _batch(dsa, T=0, max_q=0)
    assert lib.dsa_indexer_scores(ctypes.byref(empty), *args, 64, 128, FAKE, 4096, None) == dsa.DSA_OK


def test_topk_validation(dsa):
    lib = dsa.raw_lib()
    b = _batch(dsa)
    assert lib.dsa_topk(ctypes.byref(b), FAKE, 4096, 0, FAKE, None, 0, None) == dsa.DSA_ERR_UNSUPPORTED
    assert lib.dsa_topk(ctypes.byref(b), FAKE, 4096, 2049, FAKE, None, 0, None) == dsa.DSA_ERR_UNSUPPORTED
    assert lib.dsa_topk(ctypes.byref(b), None, 4096, 2048, FAKE, None, 0, None) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_topk(ctypes.byref(b), FAKE, 100, 2048, FAKE, None, 0, None) == dsa.DSA_ERR_INVALID_ARG
    long = _batch(dsa, T=8, N=8 * 131072, B=8, max_q=1, max_kv=131072)
    assert lib.dsa_topk(ctypes.byref(long), FAKE, 131072, 2048, FAKE, None, 0, None) == dsa.DSA_ERR_WORKSPACE
    need = lib.dsa_workspace_size(dsa.WS_TOPK, ctypes.byref(long), 2048, 128, 512)
    assert lib.dsa_topk(ctypes.byref(long), FAKE, 131072, 2048, FAKE, FAKE, need - 1, None) == dsa.DSA_ERR_WORKSPACE
    huge = _batch(dsa, T=1, N=300000, B=1, max_q=1, max_kv=300000)
    assert lib.dsa_topk(ctypes.byref(huge), FAKE, 300000, 2048, FAKE, FAKE, 1 << 40, None) == dsa.DSA_ERR_UNSUPPORTED


def test_sparse_mla_validation(dsa):
    lib = dsa.raw_lib()
    b = _batch(dsa)
    ok = dict(H=128, D=576, Dv=512)

    def call(q=FAKE, kv=FAKE, idx=FAKE, k=2048, H=128, D=576, Dv=512, scale=0.04, out=FAKE,
             lse=FAKE, ws=None, nbytes=0, batch=b):
        return lib.dsa_sparse_mla_fwd(ctypes.byref(batch), q, kv, idx, k, H, D, Dv, scale, out,
                                      lse, ws, nbytes, None)

    assert call(H=64) == dsa.DSA_ERR_UNSUPPORTED
    assert call(D=512) == dsa.DSA_ERR_UNSUPPORTED
    assert call(Dv=576) == dsa.DSA_ERR_UNSUPPORTED
    assert call(k=4096) == dsa.DSA_ERR_UNSUPPORTED
    assert call(q=None) == dsa.DSA_ERR_INVALID_ARG
    assert call(out=FAKE + 2) == dsa.DSA_ERR_INVALID_ARG
    assert call(scale=float("nan")) == dsa.DSA_ERR_INVALID_ARG
    dec = _batch(dsa, T=64, N=64 * 20000, B=64, max_q=1, max_kv=20000)
    assert call(batch=dec) == dsa.DSA_ERR_WORKSPACE
    assert ok


def test_dense_mla_validation(dsa):
    lib = dsa.raw_lib()
    b = _batch(dsa, 2048, 2048)

    def call(q=FAKE, kv=FAKE, H=128, D=576, Dv=512, scale=0.04, out=FAKE, lse=FAKE, ws=None, nbytes=0,
             batch=b):
        return lib.dsa_dense_mla_fwd(ctypes.byref(batch) if batch is not None else None, q, kv, H, D, Dv,
                                     scale, out, lse, ws, nbytes, None)

    assert call(batch=None) == dsa.DSA_ERR_INVALID_ARG
    assert call(H=64) == dsa.DSA_ERR_UNSUPPORTED
    assert call(D=512) == dsa.DSA_ERR_UNSUPPORTED
    assert call(batch=_batch(dsa, 4096, 4096)) == dsa.DSA_ERR_UNSUPPORTED   # longer than the short mode
    assert call(q=None) == dsa.DSA_ERR_INVALID_ARG
    assert call(kv=None) == dsa.DSA_ERR_INVALID_ARG
    assert call(lse=FAKE + 4) == dsa.DSA_ERR_INVALID_ARG
    assert call(scale=float("inf")) == dsa.DSA_ERR_INVALID_ARG
    # few rows: split-KV partials need a workspace
    few = _batch(dsa, T=4, N=4 * 2048, B=4, max_q=1, max_kv=2048)
    need = lib.dsa_workspace_size(dsa.WS_DENSE_MLA, ctypes.byref(few), 1, 128, 512)
    assert need > 0
    assert call(batch=few) == dsa.DSA_ERR_WORKSPACE
    assert call(batch=few, ws=FAKE, nbytes=need - 1) == dsa.DSA_ERR_WORKSPACE
    assert lib.dsa_workspace_size(dsa.WS_DENSE_MLA, ctypes.byref(b), 1, 128, 512) == 0
    assert lib.dsa_workspace_size(dsa.WS_DENSE_MLA, ctypes.byref(_batch(dsa, 4, 4096, max_kv=4096)), 1, 128,
                                  512) == 0


def test_indexer_kl_validation(dsa):
    lib = dsa.raw_lib()
    b = _batch(dsa, 4096, 4096)
    need = lib.dsa_workspace_size(dsa.WS_INDEXER_KL, ctypes.byref(b), 2048, 128, 512)
    assert need >= 4096 * 5 * 4

    def call(q=FAKE, kv=FAKE, lse=FAKE, H=128, D=576, scale=0.04, scores=FAKE, ld=4096, idx=FAKE, k=2048,
             kl=FAKE, p_out=None, ws=FAKE, nbytes=need, batch=b):
        return lib.dsa_indexer_kl_fwd(ctypes.byref(batch) if batch is not None else None, q, kv, lse, H, D, scale,
                                      scores, ld, idx, k, kl, p_out, ws, nbytes, None)

    assert call(batch=None) == dsa.DSA_ERR_INVALID_ARG
    assert call(H=64) == dsa.DSA_ERR_UNSUPPORTED
    assert call(D=512) == dsa.DSA_ERR_UNSUPPORTED
    assert call(k=0) == dsa.DSA_ERR_UNSUPPORTED
    assert call(k=4096) == dsa.DSA_ERR_UNSUPPORTED
    huge = _batch(dsa, 4, 3 << 21, B=1, max_kv=3 << 21)
    assert call(batch=huge, ld=3 << 21) == dsa.DSA_ERR_UNSUPPORTED
    assert call(q=None) == dsa.DSA_ERR_INVALID_ARG
    assert call(lse=None) == dsa.DSA_ERR_INVALID_ARG
    assert call(scores=None) == dsa.DSA_ERR_INVALID_ARG
    assert call(kl=None) == dsa.DSA_ERR_INVALID_ARG
    assert call(ld=4095) == dsa.DSA_ERR_INVALID_ARG
    assert call(p_out=FAKE + 4) == dsa.DSA_ERR_INVALID_ARG
    assert call(scale=float("nan")) == dsa.DSA_ERR_INVALID_ARG
    assert call(ws=None, nbytes=0) == dsa.DSA_ERR_WORKSPACE
    assert call(nbytes=need - 1) == dsa.DSA_ERR_WORKSPACE
    # the sparse attention shares the 2^21-row context limit of the gathers
    assert lib.dsa_sparse_mla_fwd(ctypes.byref(huge), FAKE, FAKE, FAKE, 2048, 128, 576, 512, 0.04, FAKE, FAKE,
                                  None, 0, None) == dsa.DSA_ERR_UNSUPPORTED


def test_sparse_mla_bwd_validation(dsa):
    lib = dsa.raw_lib()
    b = _batch(dsa, 4096, 4096)
    need = lib.dsa_workspace_size(dsa.WS_SPARSE_MLA_BWD, ctypes.byref(b), 2048, 128, 512)
    assert need >= 4096 * 2048 * (2 * 128 * 2 + 576 * 2 + 4)

    def call(q=FAKE, kv=FAKE, idx=FAKE, k=2048, H=128, D=576, Dv=512, scale=0.04, out=FAKE, lse=FAKE,
             dout=FAKE, dq=FAKE, dkv=FAKE, ws=FAKE, nbytes=need, batch=b):
        return lib.dsa_sparse_mla_bwd(ctypes.byref(batch) if batch is not None else None, q, kv, idx, k, H, D, Dv,
                                      scale, out, lse, dout, dq, dkv, ws, nbytes, None)

    assert call(batch=None) == dsa.DSA_ERR_INVALID_ARG
    assert call(H=64) == dsa.DSA_ERR_UNSUPPORTED
    assert call(Dv=576) == dsa.DSA_ERR_UNSUPPORTED
    assert call(k=0) == dsa.DSA_ERR_UNSUPPORTED
    assert call(k=4096) == dsa.DSA_ERR_UNSUPPORTED
    assert call(batch=_batch(dsa, 4, 3 << 21, max_kv=3 << 21)) == dsa.DSA_ERR_UNSUPPORTED
    for name in ("q", "kv", "idx", "out", "lse", "dout", "dq", "dkv"):
        assert call(**{name: None}) == dsa.DSA_ERR_INVALID_ARG, name
        assert call(**{name: FAKE + 8}) == dsa.DSA_ERR_INVALID_ARG, name
    assert call(scale=float("nan")) == dsa.DSA_ERR_INVALID_ARG
    assert call(ws=None, nbytes=0) == dsa.DSA_ERR_WORKSPACE
    assert call(nbytes=need - 1) == dsa.DSA_ERR_WORKSPACE


def test_fused_validation(dsa):
    lib = dsa.raw_lib()
    b = _batch(dsa)
    a = dsa.dsa_fwd_args(b, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 64, 128, 128, 576, 512, 2048, 0.04)
    for fn in (lib.dsa_prefill_fwd, lib.dsa_decode_fwd):
        assert fn(None, FAKE, FAKE, None, FAKE, 1 << 40, None) == dsa.DSA_ERR_INVALID_ARG
        assert fn(ctypes.byref(a), FAKE, FAKE, None, None, 0, None) == dsa.DSA_ERR_WORKSPACE
        need = lib.dsa_workspace_size(dsa.WS_PREFILL, ctypes.byref(b), 2048, 128, 512)
        assert fn(ctypes.byref(a), FAKE, FAKE, None, FAKE, need - 1, None) == dsa.DSA_ERR_WORKSPACE
        bad = dsa.dsa_fwd_args(b, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 64, 128, 64, 576, 512, 2048, 0.04)
        assert fn(ctypes.byref(bad), FAKE, FAKE, None, FAKE, 1 << 40, None) == dsa.DSA_ERR_UNSUPPORTED
        bad = dsa.dsa_fwd_args(b, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 64, 128, 128, 576, 512, 2048, 0.04)
        assert fn(ctypes.byref(bad), FAKE, FAKE, None, FAKE, 1 << 40, None) == dsa.DSA_ERR_INVALID_ARG
        assert fn(ctypes.byref(a), FAKE, FAKE, FAKE + 8, FAKE, 1 << 40, None) == dsa.DSA_ERR_INVALID_ARG


def test_tiny_fp32_configuration_is_unsupported(dsa):
    # the 4-head / 32-dim / 80-dim fp32 configuration is oracle-only
    lib = dsa.raw_lib()
    b = _batch(dsa, 256, 256)
    a = dsa.dsa_fwd_args(b, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 32, 8, 80, 64, 32, 80 ** -0.5)
    assert lib.dsa_prefill_fwd(ctypes.byref(a), FAKE, FAKE, None, FAKE, 1 << 40, None) == dsa.DSA_ERR_UNSUPPORTED


def test_quantize_and_append_validation(dsa):
    lib = dsa.raw_lib()
    # queries: shape support, null / misaligned pointers, empty input
    assert lib.dsa_quantize_queries(FAKE, 4, 32, 128, FAKE, FAKE, None) == dsa.DSA_ERR_UNSUPPORTED
    assert lib.dsa_quantize_queries(FAKE, 4, 64, 64, FAKE, FAKE, None) == dsa.DSA_ERR_UNSUPPORTED
    assert lib.dsa_quantize_queries(None, 4, 64, 128, FAKE, FAKE, None) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_quantize_queries(FAKE, 4, 64, 128, FAKE + 8, FAKE, None) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_quantize_queries(FAKE, -1, 64, 128, FAKE, FAKE, None) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_quantize_queries(None, 0, 64, 128, None, None, None) == dsa.DSA_OK
    # cache append
    assert lib.dsa_append_cache(FAKE, FAKE, 4, 64, 576, FAKE, FAKE, FAKE, FAKE, 100, None) == dsa.DSA_ERR_UNSUPPORTED
    assert lib.dsa_append_cache(FAKE, FAKE, 4, 128, 512, FAKE, FAKE, FAKE, FAKE, 100, None) == dsa.DSA_ERR_UNSUPPORTED
    assert lib.dsa_append_cache(FAKE, FAKE, 4, 128, 576, None, FAKE, FAKE, FAKE, 100, None) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_append_cache(FAKE, None, 4, 128, 576, FAKE, FAKE, FAKE, FAKE, 100, None) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_append_cache(FAKE, FAKE, 4, 128, 576, FAKE, FAKE, FAKE + 4, FAKE, 100, None) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_append_cache(FAKE, FAKE, -1, 128, 576, FAKE, FAKE, FAKE, FAKE, 100, None) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_append_cache(None, None, 0, 128, 576, None, None, None, None, 0, None) == dsa.DSA_OK


@pytest.mark.parametrize("scale", [0.0, -0.04, -0.0, float("-inf")])
def test_softmax_scale_must_be_positive(dsa, scale):
    """Every entry that takes the attention's softmax scale rejects scale <= 0
    (and non-finite) before launching: the kernels take max(raw logit) * scale
    as the maximum of the scaled logits, and a masked slot's -inf logit times
    such a scale is NaN or +inf."""
    lib = dsa.raw_lib()
    b = _batch(dsa, 4096, 4096)
    big = 1 << 40
    assert lib.dsa_sparse_mla_fwd(ctypes.byref(b), FAKE, FAKE, FAKE, 2048, 128, 576, 512, scale, FAKE, FAKE,
                                  FAKE, big, None) == dsa.DSA_ERR_INVALID_ARG
    s = _batch(dsa, 2048, 2048)
    assert lib.dsa_dense_mla_fwd(ctypes.byref(s), FAKE, FAKE, 128, 576, 512, scale, FAKE, FAKE, FAKE, big,
                                 None) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_indexer_kl_fwd(ctypes.byref(b), FAKE, FAKE, FAKE, 128, 576, scale, FAKE, 4096, FAKE, 2048,
                                  FAKE, None, FAKE, big, None) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_sparse_mla_bwd(ctypes.byref(b), FAKE, FAKE, FAKE, 2048, 128, 576, 512, scale, FAKE, FAKE,
                                  FAKE, FAKE, FAKE, FAKE, big, None) == dsa.DSA_ERR_INVALID_ARG
    a = dsa.dsa_fwd_args(b, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 64, 128, 128, 576, 512, 2048, scale)
    for fn in (lib.dsa_prefill_fwd, lib.dsa_decode_fwd):
        assert fn(ctypes.byref(a), FAKE, FAKE, None, FAKE, big, None) == dsa.DSA_ERR_INVALID_ARG
    # the same calls with a positive scale pass validation up to the launch
    # (which then needs a GPU): only the scale differs
    a_ok = dsa.dsa_fwd_args(b, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 64, 128, 128, 576, 512, 2048, 0.04)
    assert lib.dsa_prefill_fwd(ctypes.byref(a_ok), FAKE, FAKE, FAKE + 8, FAKE, big, None) == dsa.DSA_ERR_INVALID_ARG


def test_profile_entry_validation(dsa):
    lib = dsa.raw_lib()
    b = _batch(dsa)
    a = dsa.dsa_fwd_args(b, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 64, 128, 128, 576, 512, 2048, 0.04)
    n = ctypes.c_int(-1)
    times = (dsa.dsa_kernel_time * 4)()
    assert lib.dsa_fwd_profile(ctypes.byref(a), 0, FAKE, FAKE, None, FAKE, 1 << 40, None, None, 4,
                               ctypes.byref(n)) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_fwd_profile(ctypes.byref(a), 0, FAKE, FAKE, None, FAKE, 1 << 40, None, times, 0,
                               ctypes.byref(n)) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_fwd_profile(ctypes.byref(a), 0, FAKE, FAKE, None, FAKE, 1 << 40, None, times, 4,
                               None) == dsa.DSA_ERR_INVALID_ARG


def test_log_lines(dsa, capfd, monkeypatch):
    """DSA_LOG=1: one stderr line per call with the batch, k, workspace and
    status (read at every call); nothing without it."""
    lib = dsa.raw_lib()
    b = _batch(dsa)
    monkeypatch.delenv("DSA_LOG", raising=False)
    assert lib.dsa_topk(ctypes.byref(b), None, 4096, 2048, FAKE, None, 0, None) == dsa.DSA_ERR_INVALID_ARG
    assert "[dsa]" not in capfd.readouterr().err
    monkeypatch.setenv("DSA_LOG", "1")
    assert lib.dsa_topk(ctypes.byref(b), None, 4096, 2048, FAKE, None, 0, None) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_prefill_fwd(None, FAKE, FAKE, None, None, 0, None) == dsa.DSA_ERR_INVALID_ARG
    err = capfd.readouterr().err
    assert "[dsa] dsa_topk B=1 total_q=4096 max_q=4096 max_kv=4096 total_kv=4096 k=2048 ws=0 -> invalid argument" \
        in err, err
    assert "[dsa] dsa_prefill_fwd -> invalid argument" in err, err
    monkeypatch.setenv("DSA_LOG", "0")
    assert lib.dsa_topk(ctypes.byref(b), None, 4096, 2048, FAKE, None, 0, None) == dsa.DSA_ERR_INVALID_ARG
    assert "[dsa]" not in capfd.readouterr().err


def test_check_selection_validation(dsa):
    lib = dsa.raw_lib()
    b = _batch(dsa)
    bad = ctypes.c_int(-7)
    assert lib.dsa_check_selection(ctypes.byref(b), FAKE, 2048, None, None) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_check_selection(ctypes.byref(b), None, 2048, None, ctypes.byref(bad)) == dsa.DSA_ERR_INVALID_ARG
    assert bad.value == 0
    assert lib.dsa_check_selection(ctypes.byref(b), FAKE + 4, 2048, None, ctypes.byref(bad)) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_check_selection(ctypes.byref(b), FAKE, 0, None, ctypes.byref(bad)) == dsa.DSA_ERR_UNSUPPORTED
    assert lib.dsa_check_selection(None, FAKE, 2048, None, ctypes.byref(bad)) == dsa.DSA_ERR_INVALID_ARG
    empty = _batch(dsa, T=0, N=10, max_q=0, max_kv=10)
    assert lib.dsa_check_selection(ctypes.byref(empty), None, 16, None, ctypes.byref(bad)) == dsa.DSA_OK


def test_measure_peaks_validation(dsa):
    # argument checks come before any GPU call: no device needed
    lib = dsa.raw_lib()
    r = dsa.dsa_peaks()
    big = 256 << 20
    assert lib.dsa_measure_peaks(None, big, None, ctypes.byref(r)) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_measure_peaks(FAKE, big, None, None) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_measure_peaks(FAKE + 4, big, None, ctypes.byref(r)) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_measure_peaks(FAKE, (64 << 20) - 16, None, ctypes.byref(r)) == dsa.DSA_ERR_INVALID_ARG
