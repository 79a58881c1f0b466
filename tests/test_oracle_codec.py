"""Pins for the oracle's FP8 E4M3FN and bf16 decoders, and for the input
generator's quantiser.  The decoders follow the OCP FP8 and bf16 bit layouts;
they are checked against closed-form values and torch's own casts."""
import math

import numpy as np
import torch

import oracle
import synth


def test_e4m3_closed_form_values():
    # OCP E4M3FN: bias 7, 3 mantissa bits, max 448, S.1111.111 = NaN
    cases = {
        0x00: 0.0, 0x38: 1.0, 0x40: 2.0, 0x30: 0.5, 0x3C: 1.5,
        0x7E: 448.0, 0xFE: -448.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9,
        0x08: 2.0 ** -6, 0xB8: -1.0, 0x77: 240.0, 0x78: 256.0,
    }
    for code, v in cases.items():
        assert oracle.e4m3_value(code) == v, hex(code)
    assert math.copysign(1.0, oracle.e4m3_value(0x80)) == -1.0 and oracle.e4m3_value(0x80) == 0.0
    assert math.isnan(oracle.e4m3_value(0x7F)) and math.isnan(oracle.e4m3_value(0xFF))


def test_e4m3_table_matches_torch_cast():
    tab = oracle.e4m3_table()
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(tab), nan)
    assert np.array_equal(tab[~nan], ref[~nan])
    # every finite code is distinct except +-0, and the finite set is symmetric
    fin = tab[~nan]
    assert len(set(fin.tolist())) == 253
    assert np.array_equal(np.sort(fin[fin > 0]), np.sort(-fin[fin < 0]))


def test_bf16_matches_torch_cast():
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 1 << 16, size=4096, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    got = np.array([oracle.bf16_value(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert oracle.bf16_value(0x3F80) == 1.0 and oracle.bf16_value(0xC000) == -2.0


def test_generator_quantiser_round_trip():
    # codes * scale reproduce x within half an E4M3 step; absmax maps to +-448
    x = synth.normal_rows(7, 99, 0, 64, 128)
    codes, scale = synth.quant_e4m3_rows(x)
    tab = oracle.e4m3_table()
    deq = tab[codes] * scale[:, None].astype(np.float64)
    amax = np.abs(x).max(axis=1)
    # relative step of E4M3 is 2^-3 in the normal range -> rounding error <= 2^-4 relative,
    # plus the subnormal absolute step 2^-9 * scale
    err = np.abs(deq - x)
    bound = np.abs(x) * 2.0 ** -4 + (2.0 ** -10) * scale[:, None] + 1e-12
    assert np.all(err <= bound)
    top = np.abs(tab[codes]).max(axis=1)
    assert np.all(top == 448.0)
    assert np.allclose(scale, amax / 448.0, rtol=1e-7)


def test_generator_is_block_addressable():
    full = synth.normal_rows(11, 5, 0, 3000, 128)
    part = synth.normal_rows(11, 5, 1234, 2101, 128)
    assert np.array_equal(full[1234:2101], part)
    other = synth.normal_rows(12, 5, 0, 10, 128)
    assert not np.array_equal(full[:10], other)
