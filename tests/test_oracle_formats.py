"""Pins of oracle.formats against an independent library routine
(torch.float8_e4m3fn) and the E2M1 bit-level definition."""
import numpy as np
import pytest
import torch

from oracle import formats as F


def _torch_e4m3(x32):
    return torch.from_numpy(np.asarray(x32, dtype=np.float32)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()


def test_e4m3_decode_all_bytes_match_torch():
    b = np.arange(256, dtype=np.uint8)
    ours = F.e4m3_decode(b)
    ref = torch.from_numpy(b).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert F.E4M3_POS[-1] == 448.0 and len(F.E4M3_POS) == 127
    assert np.all(np.diff(F.E4M3_POS) > 0)


def test_e4m3_encode_random_matches_torch():
    rng = np.random.default_rng(123)
    mag = np.exp2(rng.uniform(-13, np.log2(463.0), 200000))
    x = (mag * rng.choice([-1.0, 1.0], mag.size)).astype(np.float32)
    assert np.array_equal(F.e4m3_encode(x.astype(np.float64)), _torch_e4m3(x))


def test_e4m3_encode_midpoints_and_neighbours_match_torch():
    mids = F.E4M3_MID.astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), F.E4M3_MID)     # exact in fp32
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(0))
    for arr in (mids, up, dn, -mids, -up, -dn, F.E4M3_POS.astype(np.float32)):
        assert np.array_equal(F.e4m3_encode(arr.astype(np.float64)), _torch_e4m3(arr))


def test_e4m3_encode_ties_go_to_even_code():
    # e.g. 17 lies between 16 (0x58) and 18 (0x59): the even code wins
    assert F.e4m3_encode(17.0) == 0x58
    # 2^-10 lies between 0 and the smallest subnormal 2^-9: rounds to +0
    assert F.e4m3_encode(2.0 ** -10) == 0x00
    assert F.e4m3_encode(-(2.0 ** -10)) == 0x80                      # sign kept


def test_e4m3_encode_saturates():
    assert F.e4m3_encode(448.0) == 0x7E
    assert F.e4m3_encode(463.99) == 0x7E
    assert F.e4m3_encode(1e6) == 0x7E
    assert F.e4m3_encode(-1e6) == 0xFE


def test_e2m1_table_from_bit_definition():
    # E2M1: 2 exponent bits (bias 1), 1 mantissa bit, subnormal when exponent is 0
    vals = []
    for code in range(8):
        e, m = code >> 1, code & 1
        vals.append(m * 0.5 if e == 0 else (1 + m / 2) * 2.0 ** (e - 1))
    assert np.array_equal(F.E2M1_MAG, np.array(vals))


@pytest.mark.parametrize("a,expect", [
    (0.25, 0), (0.2500001, 1), (0.75, 2), (0.7499999, 1), (1.25, 2), (1.2500001, 3),
    (1.75, 4), (2.5, 4), (2.5000002, 5), (3.5, 6), (3.4999998, 5), (5.0, 6), (5.0000005, 7),
    (6.0, 7), (100.0, 7), (0.0, 0),
])
def test_nearest_even_index_e2m1_hand_cases(a, expect):
    assert int(F.nearest_even_index(np.float64(np.float32(a)), F.E2M1_MID)) == expect
