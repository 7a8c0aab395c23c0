"""Pins of the oracle's E4M3FN codec against the format definition and torch's cast."""
import numpy as np
import pytest
import torch

from oracle import e4m3


def torch_encode(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def torch_decode(codes):
    return torch.from_numpy(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_special_codes_from_format_definition():
    d = e4m3.DECODE_TABLE
    assert d[0x00] == 0.0 and not np.signbit(d[0x00])
    assert d[0x80] == 0.0 and np.signbit(d[0x80])
    assert d[0x01] == 2.0 ** -9          # smallest subnormal
    assert d[0x07] == 7 * 2.0 ** -9      # largest subnormal
    assert d[0x08] == 2.0 ** -6          # smallest normal
    assert d[0x38] == 1.0
    assert d[0x3C] == 1.5
    assert d[0x7E] == 448.0              # largest finite
    assert d[0xFE] == -448.0
    assert np.isnan(d[0x7F]) and np.isnan(d[0xFF])
    finite = d[np.isfinite(d)]
    assert finite.size == 254
    assert np.unique(finite).size == 253   # +0 and -0 compare equal


def test_decode_matches_torch_for_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours, ref = e4m3.decode(codes), torch_decode(codes)
    np.testing.assert_array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(ours[ok], ref[ok])


def test_round_trip_every_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    np.testing.assert_array_equal(e4m3.encode(e4m3.decode(codes)), codes)


def test_ties_round_to_even():
    # 1.0625 lies halfway between 1.0 (mantissa 000) and 1.125 (001): even wins.
    assert e4m3.encode(np.array([1.0625]))[0] == 0x38
    # 1.1875 halfway between 1.125 (001) and 1.25 (010): even wins -> 1.25.
    assert e4m3.round_to_grid(np.array([1.1875]))[0] == 1.25
    # subnormal ties: 2^-10 -> 0, 3*2^-10 -> 2*2^-9
    assert e4m3.round_to_grid(np.array([2.0 ** -10]))[0] == 0.0
    assert e4m3.round_to_grid(np.array([3 * 2.0 ** -10]))[0] == 2 * 2.0 ** -9
    # the tie just above the largest subnormal goes to the smallest normal (even mantissa)
    assert e4m3.round_to_grid(np.array([7.5 * 2.0 ** -9]))[0] == 2.0 ** -6


def test_saturation_and_nan():
    out = e4m3.encode(np.array([448.0, 449.0, 1000.0, -1e9, np.nan]))
    assert list(out) == [0x7E, 0x7E, 0x7E, 0xFE, 0x7F]


@pytest.mark.parametrize("seed", [0, 1])
def test_encode_matches_torch_dense_sweep(seed):
    rng = np.random.default_rng(seed)
    grid = e4m3.DECODE_TABLE[np.isfinite(e4m3.DECODE_TABLE)]
    grid = np.unique(grid)
    mids = (grid[1:] + grid[:-1]) / 2                # every tie
    x = np.concatenate([grid, mids, np.nextafter(mids, np.inf), np.nextafter(mids, -np.inf),
                        rng.uniform(-448, 448, 20000), rng.uniform(-0.05, 0.05, 20000)])
    x = x.astype(np.float32).astype(np.float64)      # torch casts from float32
    np.testing.assert_array_equal(e4m3.encode(x), torch_encode(x))
