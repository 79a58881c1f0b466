"""The allocation-free decode entry (dsa_decode_fwd_noalloc: the same decode
path on the library's static scratch) against dsa_decode_fwd with a caller
workspace: out, lse and idx identical bit for bit, on two calls in a row (the
second on a smaller batch, so it runs over what the first left in the scratch),
called through the C ABI.  A batch larger than the scratch is refused before
any launch."""
import ctypes

import numpy as np
import pytest
import torch

import synth
from gpu_util import DevInputs, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsa():
    import sparse_attention_16_amd as m  # fails loudly when libdsa.so is missing
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def _check(dsa, inp, what):
    b = inp.batch
    d = DevInputs(inp, dsa)
    args = dsa.fwd_args(d.batch, d.qi, d.qs, d.w, d.ki, d.ks, d.q, d.kv, inp.k, inp.scale)
    out = torch.empty((b.T, inp.H, inp.Dv), dtype=torch.int16, device="cuda")
    lse = torch.empty((b.T, inp.H), device="cuda")
    idx = torch.empty((b.T, inp.k), dtype=torch.int32, device="cuda")
    dsa.decode_fwd(args, d.batch, out, lse, idx)
    out2 = torch.full_like(out, -1)
    lse2 = torch.full_like(lse, float("nan"))
    idx2 = torch.full_like(idx, -9)
    lib = dsa.raw_lib()
    st = lib.dsa_decode_fwd_noalloc(ctypes.byref(args), out2.data_ptr(), lse2.data_ptr(), idx2.data_ptr(),
                                    torch.cuda.current_stream().cuda_stream)
    assert st == dsa.DSA_OK, dsa.status_string(st)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2), f"{what}: idx differs"
    assert torch.equal(out, out2), f"{what}: out differs"
    assert torch.equal(lse.view(torch.int32), lse2.view(torch.int32)), f"{what}: lse differs"
    say(f"  {what}: {b.T} rows, out / lse / idx identical to dsa_decode_fwd")


def test_noalloc_decode_matches_decode_fwd(dsa):
    say("[decode_fwd_noalloc] two calls, the second smaller")
    need_max = dsa.raw_lib().dsa_decode_fwd_noalloc_max_bytes()
    assert need_max == 128 << 20
    ctx1 = synth.decode_contexts(0xD5B0, 24, 2000, 70000)
    ctx1[:3] = [1, 2048, 40000]
    big = synth.make_inputs(synth.Batch.decode(ctx1), seed=171, k=2048, per_seq=True)
    b1 = dsa.Batch.from_host(big.batch.cu_q, big.batch.cu_kv, big.batch.pos0)
    assert 0 < dsa.workspace_size(dsa.WS_DECODE, b1, 2048) <= need_max
    _check(dsa, big, "first call: 24 sequences up to 70000 keys")
    small = synth.make_inputs(synth.Batch.decode([3, 5000, 33000]), seed=172, k=2048, per_seq=True)
    _check(dsa, small, "second call: 3 sequences")


def test_noalloc_decode_refuses_oversized_batch(dsa):
    # 64 sequences of 262144 keys need more than the static scratch: refused
    # on the host (no device data is touched, so the pointers may be fake)
    fake = 1 << 20
    n = 262144
    batch = dsa.dsa_batch(64, 64, 1, n, 64 * n, fake, fake, fake)
    args = dsa.dsa_fwd_args(batch, fake, fake, fake, fake, fake, fake, fake, 64, 128, 128, 576, 512, 2048, 0.04)
    st = dsa.raw_lib().dsa_decode_fwd_noalloc(ctypes.byref(args), fake, fake, None, None)
    assert st == dsa.DSA_ERR_WORKSPACE
