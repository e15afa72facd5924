"""Pins of the oracle's number formats against the formats' definitions and
torch's CPU casts (a library routine independent of the oracle)."""
import struct

import numpy as np
import torch

from oracle import numerics as nx


def test_bf16_widen_is_top_half_of_binary32():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 16, 4000, dtype=np.int64).astype(np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]               # finite only
    got = nx.bf16_to_f64(bits)
    for b, g in zip(bits[:500], got[:500]):
        want = struct.unpack("<f", struct.pack("<I", int(b) << 16))[0]
        assert g == want


def test_f32_to_bf16_matches_torch_round_to_nearest_even():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(20000).astype(np.float32) * 3
    # exact midpoints between neighbouring bf16 values, both parities
    mids = ((rng.integers(0, 1 << 15, 2000).astype(np.uint32) << 16) | 0x8000).view(np.float32)
    mids = mids[np.isfinite(mids)]
    x = np.concatenate([x, mids, np.float32([0.0, -0.0, 1.0, 65504.0, 1e-30])])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(nx.f32_to_bf16(x), want)


def test_e4m3_table_matches_torch_float8_e4m3fn():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    want = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = nx.E4M3_VALUES
    nan = np.isnan(want)
    assert np.array_equal(nan, np.isnan(got))
    np.testing.assert_array_equal(got[~nan], want[~nan])
    assert nx.E4M3_VALUES[0x7E] == 448.0 and nx.E4M3_VALUES[0x01] == 2.0 ** -9


def test_e4m3_all_codes_round_trip():
    for c in range(256):
        v = nx.E4M3_VALUES[c]
        if np.isnan(v):
            continue
        back = int(nx.e4m3_encode(np.array([v]))[0])
        if v == 0.0:
            assert back == 0
        else:
            assert back == c, (c, v, back)


def test_e4m3_midpoints_round_to_even_code():
    vals = nx.E4M3_VALUES[:127]
    for c in range(126):
        mid = 0.5 * (vals[c] + vals[c + 1])
        got = int(nx.e4m3_encode(np.array([mid]))[0])
        assert got == (c if c % 2 == 0 else c + 1), (c, mid, got)
        # just off the midpoint goes to the nearer neighbour
        assert int(nx.e4m3_encode(np.array([np.nextafter(mid, 0)]))[0]) == c
        assert int(nx.e4m3_encode(np.array([np.nextafter(mid, 1e9)]))[0]) == c + 1


def test_e4m3_encode_matches_torch_in_range_and_saturates_beyond():
    rng = np.random.default_rng(2)
    x = np.concatenate([rng.standard_normal(20000) * 40, rng.uniform(-464, 464, 5000),
                        rng.standard_normal(2000) * 1e-3]).astype(np.float32)
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(nx.e4m3_round(x.astype(np.float64)), want)
    big = np.array([448.0, 449.0, 500.0, 1e6, -1e6])
    np.testing.assert_array_equal(nx.e4m3_round(big), [448.0, 448.0, 448.0, 448.0, -448.0])
