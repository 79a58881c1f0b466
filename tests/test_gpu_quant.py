"""GPU parity of the FP8 quantise and cache-append entry points
(dsa_quantize_queries, dsa_append_cache) against the oracle quantiser:
codes and scales bit-exact, latent rows copied exactly, untouched cache rows
unchanged.  The quantisation is the step before the index score (page
"Техотчёт DeepSeek-V3.2 (2025): разреженное внимание DSA и масштабирование
RL", section "Молниеносный индексатор")."""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

HI, DI, D = 64, 128, 576


@pytest.fixture(scope="module")
def dsa():
    import sparse_attention_16_amd as m  # fails loudly when libdsa.so is missing
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def e4m3_values_and_midpoints():
    tab = oracle.e4m3_table()
    pos = np.array(sorted(set(tab[c] for c in range(256) if not np.isnan(tab[c]) and tab[c] >= 0)))
    mids = (pos[:-1] + pos[1:]) / 2
    return np.concatenate([pos, mids, -pos, -mids]).astype(np.float32)


def query_cases(T, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, HI * DI)).astype(np.float32)
    q *= rng.uniform(1e-3, 1e3, (T, 1)).astype(np.float32)
    if T > 4:
        q[1] = 0.0                                       # all-zero token: scale 1, codes 0
        q[2] *= np.float32(1e-30)                        # tiny magnitudes
        q[3] *= np.float32(1e30)                         # huge magnitudes
        v = e4m3_values_and_midpoints()                  # absmax 448: scale 1, exact ties
        q[4] = 0.0
        q[4, :v.size] = v
    return q


@pytest.mark.parametrize("T", [1, 5, 37, 300])
def test_quantize_queries_bit_exact(dsa, T):
    q = query_cases(T, seed=100 + T)
    codes_ref, scale_ref = oracle.quant_rows(q)
    qd = torch.from_numpy(q).reshape(T, HI, DI).cuda()
    codes = torch.empty((T, HI, DI), dtype=torch.uint8, device="cuda")
    scale = torch.empty((T, HI), dtype=torch.float32, device="cuda")
    dsa.quantize_queries(qd, codes, scale)
    torch.cuda.synchronize()
    assert np.array_equal(codes.cpu().numpy().reshape(T, HI * DI), codes_ref)
    s = scale.cpu().numpy()
    assert np.array_equal(s, np.repeat(scale_ref[:, None], HI, axis=1))


def test_quantize_queries_full_size_sampled(dsa):
    T = 32768
    rng = np.random.default_rng(7)
    qd = torch.randn((T, HI, DI), dtype=torch.float32, device="cuda", generator=torch.Generator("cuda").manual_seed(7))
    codes = torch.empty((T, HI, DI), dtype=torch.uint8, device="cuda")
    scale = torch.empty((T, HI), dtype=torch.float32, device="cuda")
    dsa.quantize_queries(qd, codes, scale)
    torch.cuda.synchronize()
    rows = np.sort(rng.choice(T, 48, replace=False))
    rows[0], rows[-1] = 0, T - 1
    x = qd[torch.from_numpy(rows).cuda()].reshape(len(rows), HI * DI).cpu().numpy()
    codes_ref, scale_ref = oracle.quant_rows(x)
    got = codes[torch.from_numpy(rows).cuda()].reshape(len(rows), HI * DI).cpu().numpy()
    assert np.array_equal(got, codes_ref)
    assert np.array_equal(scale[torch.from_numpy(rows).cuda()].cpu().numpy(), np.repeat(scale_ref[:, None], HI, axis=1))


def run_append(dsa, N, k_new, kv_new, dst):
    sentinel_code, sentinel_scale, sentinel_kv = 0x5A, np.float32(-7.25), 0x1234
    k_fp8 = torch.full((N, DI), sentinel_code, dtype=torch.uint8, device="cuda")
    k_scale = torch.full((N,), float(sentinel_scale), dtype=torch.float32, device="cuda")
    kv = torch.full((N, D), sentinel_kv, dtype=torch.int16, device="cuda")
    kn = torch.from_numpy(k_new).cuda()
    kvn = torch.from_numpy(kv_new.view(np.int16)).cuda() if kv_new is not None else None
    dd = torch.from_numpy(dst.astype(np.int64)).cuda()
    dsa.append_cache(kn, kvn, dd, k_fp8, k_scale, kv if kv_new is not None else None)
    torch.cuda.synchronize()
    codes_ref, scale_ref = oracle.quant_rows(k_new)
    got_c, got_s, got_kv = k_fp8.cpu().numpy(), k_scale.cpu().numpy(), kv.cpu().numpy().view(np.uint16)
    inside = (dst >= 0) & (dst < N)
    written = np.zeros(N, dtype=bool)
    written[dst[inside]] = True
    assert np.array_equal(got_c[dst[inside]], codes_ref[inside])
    assert np.array_equal(got_s[dst[inside]], scale_ref[inside])
    assert np.all(got_c[~written] == sentinel_code)
    assert np.all(got_s[~written] == sentinel_scale)
    if kv_new is not None:
        assert np.array_equal(got_kv[dst[inside]], kv_new[inside])
    assert np.all(got_kv[~written] == sentinel_kv)


@pytest.mark.parametrize("R,N,with_kv", [(1, 10, True), (77, 1000, True), (77, 1000, False), (513, 4096, True)])
def test_append_cache_bit_exact(dsa, R, N, with_kv):
    rng = np.random.default_rng(R * 7 + N)
    k_new = (rng.standard_normal((R, DI)) * rng.uniform(1e-2, 1e2, (R, 1))).astype(np.float32)
    if R > 3:
        k_new[2] = 0.0
        k_new[3, :64] = e4m3_values_and_midpoints()[:64]
        k_new[3, 64:] = 0.0
        k_new[3, 0] = 448.0
    kv_new = rng.integers(0, 1 << 16, (R, D), dtype=np.uint32).astype(np.uint16) if with_kv else None
    dst = rng.choice(N, R, replace=False).astype(np.int64)
    if R > 8:
        dst[5], dst[6] = -1, N + 3                       # out of range: skipped
    run_append(dsa, N, k_new, kv_new, dst)


def test_append_cache_full_size(dsa):
    # one 32768-token prefill appended behind 1000 cached rows
    R, N = 32768, 40000
    rng = np.random.default_rng(3)
    k_new = rng.standard_normal((R, DI)).astype(np.float32)
    kv_new = rng.integers(0, 1 << 16, (R, D), dtype=np.uint32).astype(np.uint16)
    dst = np.arange(1000, 1000 + R, dtype=np.int64)
    run_append(dsa, N, k_new, kv_new, dst)
