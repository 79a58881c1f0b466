"""Pins for the oracle's FP8 E4M3FN encoder and per-group absmax quantiser
(the quantise step before the index score: page "Техотчёт DeepSeek-V3.2 (2025):
разреженное внимание DSA и масштабирование RL", section "Молниеносный
индексатор", the indexer runs on FP8 values).  The encoder is an exhaustive
nearest-code search; it is pinned to torch's float8_e4m3fn cast (a library
round-to-nearest-even conversion), to the decoder (round trip over every code)
and to closed forms; the quantiser is pinned to the input generator's numpy /
torch quantiser and to its defining properties."""
import numpy as np
import torch

import oracle
import synth

TAB = oracle.e4m3_table()
FIN = [c for c in range(256) if not np.isnan(TAB[c])]


def torch_e4m3(y: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(y, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def enc(y: np.ndarray) -> np.ndarray:
    return np.array([oracle.e4m3_encode(float(v)) for v in np.asarray(y, dtype=np.float32)], dtype=np.uint8)


def test_encode_round_trips_every_code():
    for c in FIN:
        got = oracle.e4m3_encode(float(np.float32(TAB[c])))
        # +0 and -0 keep their sign; every other code is its own encoding
        assert got == c, (hex(c), hex(got))


def test_encode_matches_torch_on_midpoints_and_random_values():
    pos = np.array(sorted(set(TAB[c] for c in FIN if TAB[c] >= 0)))
    mids = (pos[:-1] + pos[1:]) / 2            # exact ties (representable in binary32)
    rng = np.random.default_rng(11)
    vals = np.concatenate([
        pos, mids, -mids,
        rng.uniform(-448, 448, 20000),
        rng.uniform(-2.0 ** -5, 2.0 ** -5, 5000),   # subnormal and smallest normals
        np.nextafter(mids, 0), np.nextafter(mids, 1000),
    ]).astype(np.float32)
    assert np.array_equal(enc(vals), torch_e4m3(vals))


def test_encode_closed_forms():
    assert oracle.e4m3_encode(1.0) == 0x38
    assert oracle.e4m3_encode(-1.0) == 0xB8
    assert oracle.e4m3_encode(2.0 ** -9) == 0x01
    assert oracle.e4m3_encode(2.0 ** -10) == 0x00      # tie between 0 and 2^-9: even code 0
    assert oracle.e4m3_encode(3 * 2.0 ** -10) == 0x02  # tie between 1 and 2 (x 2^-9): even code 2
    assert oracle.e4m3_encode(1.0625) == 0x38          # tie between 1 and 1.125: even mantissa
    assert oracle.e4m3_encode(1.1875) == 0x3A          # tie between 1.125 and 1.25: even mantissa
    for y in (448.0, 449.0, 463.9, 1e6):               # saturation at the largest finite code
        assert oracle.e4m3_encode(y) == 0x7E
        assert oracle.e4m3_encode(-y) == 0xFE
    assert oracle.e4m3_encode(-0.0) == 0x80 and oracle.e4m3_encode(0.0) == 0x00
    assert oracle.e4m3_encode(-1e-30) == 0x80


def test_quant_rows_matches_generator_quantiser():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((64, 128)).astype(np.float32)
    x[3] = 0.0                                  # all-zero group: scale 1
    x[7] *= 1e-30                               # tiny group
    x[9] *= 1e4                                 # large group
    codes, scale = oracle.quant_rows(x)
    c2, s2 = synth.quant_e4m3_rows(x)
    assert np.array_equal(scale, s2)
    assert np.array_equal(codes, c2)


def test_quant_rows_properties():
    rng = np.random.default_rng(9)
    x = (rng.standard_normal((32, 8192)) * rng.uniform(0.01, 100, (32, 1))).astype(np.float32)
    codes, scale = oracle.quant_rows(x)
    amax = np.abs(x).max(axis=1)
    assert np.array_equal(scale, (amax / np.float32(448)).astype(np.float32))
    # the largest-magnitude element of each group lands on +-448
    for r in range(32):
        i = int(np.argmax(np.abs(x[r])))
        assert codes[r, i] & 0x7F == 0x7E
    # dequantised values are within half a code spacing of x (relative 1/16 for normals)
    deq = TAB[codes] * scale[:, None]
    big = np.abs(x) >= 2.0 ** -6 * scale[:, None]
    assert np.all(np.abs(deq - x)[big] <= np.abs(x)[big] / 16 * (1 + 1e-6))
    # the sign bit is that of x
    assert np.array_equal(codes >= 0x80, np.signbit(x))
