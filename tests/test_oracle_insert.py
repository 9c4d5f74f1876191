"""Pins of oracle.insert (the cache-insertion path after the QKV projection):
bf16 decoding against torch's bfloat16, closed-form RMSNorm cases, RoPE
against a complex-number rotation and closed-form unit-vector cases, pair
norms and relative-position invariance, and where each segment of a
projection row ends up."""
import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import insert as I
from oracle import nvfp4 as N


def test_bf16_decoding_matches_torch():
    bits = np.arange(1 << 16, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    got = I.bf16_to_f64(bits)
    both_nan = np.isnan(ref) & np.isnan(got)
    assert np.array_equal(got[~both_nan], ref[~both_nan])
    assert np.array_equal(np.isnan(ref), np.isnan(got))


def test_rms_norm_closed_forms():
    rng = np.random.default_rng(0)
    x = rng.normal(size=(5, 3, 128)) * rng.uniform(0.1, 10, size=(5, 3, 1))
    y = I.rms_norm(x, np.ones(128), 0.0)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, rtol=1e-12)
    # invariant to a positive scale of the input
    assert np.allclose(I.rms_norm(7.5 * x, np.ones(128), 0.0), y, rtol=1e-12)
    # a constant row -> its sign times the weight
    w = rng.uniform(0.5, 2, size=128)
    assert np.allclose(I.rms_norm(np.full(128, -3.0), w, 0.0), -w, rtol=1e-12)
    # one non-zero channel v: mean = v^2 / 128 -> sqrt(128) at that channel
    e = np.zeros(128)
    e[17] = 0.25
    y1 = I.rms_norm(e, np.ones(128), 0.0)
    assert y1[17] == pytest.approx(np.sqrt(128.0), rel=1e-12) and np.count_nonzero(y1) == 1
    # eps enters under the root: x = 0 stays 0
    assert np.array_equal(I.rms_norm(np.zeros(128), w, 1e-6), np.zeros(128))


def _rope_complex(x, pos, r, theta):
    # rotate-half RoPE as multiplication of z_i = x_i + j x_{i+r/2} by exp(j angle_i)
    h = r // 2
    i = np.arange(h)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * theta ** (-(2.0 * i) / r)
    z = (x[..., :h] + 1j * x[..., h:r]) * np.exp(1j * ang)[:, None, :]
    y = x.copy()
    y[..., :h], y[..., h:r] = z.real, z.imag
    return y


@pytest.mark.parametrize("r,theta", [(128, 10000.0), (64, 10000.0), (32, 5e5), (96, 1e6)])
def test_rope_is_a_complex_rotation(r, theta):
    rng = np.random.default_rng(r)
    x = rng.normal(size=(6, 4, 128))
    pos = np.array([0, 1, 7, 1000, 65535, 262143])
    y = I.rope(x, pos, r, theta)
    assert np.allclose(y, _rope_complex(x, pos, r, theta), rtol=0, atol=1e-12)
    assert np.array_equal(y[..., r:], x[..., r:])          # untouched channels
    h = r // 2                                              # pair norms kept
    assert np.allclose(y[..., :h] ** 2 + y[..., h:r] ** 2, x[..., :h] ** 2 + x[..., h:r] ** 2)


def test_rope_unit_vectors_and_special_cases():
    p = 3.0
    e0 = np.zeros((1, 1, 128))
    e0[..., 0] = 1.0
    y = I.rope(e0, [p], 128, 10000.0)
    assert y[0, 0, 0] == pytest.approx(np.cos(p)) and y[0, 0, 64] == pytest.approx(np.sin(p))
    assert np.count_nonzero(np.abs(y) > 1e-15) == 2
    e64 = np.zeros((1, 1, 128))
    e64[..., 64] = 1.0
    y = I.rope(e64, [p], 128, 10000.0)
    assert y[0, 0, 0] == pytest.approx(-np.sin(p)) and y[0, 0, 64] == pytest.approx(np.cos(p))
    # frequency of pair 5: theta^(-10/128)
    e5 = np.zeros((1, 1, 128))
    e5[..., 5] = 1.0
    a = 1234.0 * 10000.0 ** (-10.0 / 128.0)
    y = I.rope(e5, [1234.0], 128, 10000.0)
    assert y[0, 0, 5] == pytest.approx(np.cos(a), abs=1e-12) and y[0, 0, 69] == pytest.approx(np.sin(a), abs=1e-12)
    x = np.random.default_rng(1).normal(size=(2, 3, 128))
    assert np.array_equal(I.rope(x, [0, 0], 128, 10000.0), x)       # position 0
    assert np.array_equal(I.rope(x, [5, 9], 0, 10000.0), x)         # no rotary channels


def test_rope_dot_products_depend_on_relative_position():
    rng = np.random.default_rng(2)
    q, k = rng.normal(size=(1, 1, 128)), rng.normal(size=(1, 1, 128))
    d0 = np.sum(I.rope(q, [100], 128, 1e4) * I.rope(k, [40], 128, 1e4))
    d1 = np.sum(I.rope(q, [5100], 128, 1e4) * I.rope(k, [5040], 128, 1e4))
    assert d0 == pytest.approx(d1, rel=1e-9)


def _bf16_bits(x):
    return torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_insert_places_each_segment():
    hkv, hidx = 2, 1
    hq, hqi = 8 * hkv, 8 * hidx
    seg = [(hq, 1.0), (hqi, 0.5), (hkv, 2.0), (hkv, 3.0), (hidx, 4.0)]
    t = 3
    row = np.concatenate([np.full(n * 128, v) for n, v in seg])
    rows = _bf16_bits(np.tile(row, (t, 1)))
    pools = [N.empty_pool(4, h, fill=0xEE) for h in (hkv, hkv, hidx)]
    slots = np.array([5, -1, 3 * 128 + 9])
    q, qi = I.insert(rows, [0, 1, 2], slots, *pools, rotary_dim=0)
    assert q.shape == (t, hq, 128) and np.all(q == F.e4m3_encode(1.0))
    assert qi.shape == (t, hqi, 128) and np.all(qi == F.e4m3_encode(0.5))
    for (codes, scales), want in zip(pools, (2.0, 3.0, 4.0)):
        for slot in (5, 3 * 128 + 9):
            _, vals = N.dequant_fp8(codes[slot // 128, :, slot % 128], scales[slot // 128, :, slot % 128])
            assert np.allclose(vals, want, rtol=0.1)
        assert np.all(codes[0, :, 6] == 0xEE)               # untouched rows
    # the skipped token (slot -1) wrote nothing: only two rows per pool changed
    for codes, _ in pools:
        assert np.count_nonzero(np.any(codes != 0xEE, axis=(1, 3))) == 2


def test_insert_norm_and_rope_reach_the_outputs():
    hkv, hidx = 1, 1
    rng = np.random.default_rng(3)
    rows = _bf16_bits(rng.normal(size=(2, (8 + 8 + 1 + 1 + 1) * 128)))
    w = np.ones(128)
    q, qi, k, v, ki = I.transform(rows, [11, 12], hkv, hidx, w, w, 0.0, 128, 1e4)
    x = I.bf16_to_f64(rows)
    assert np.allclose(np.sqrt(np.mean(k ** 2, axis=-1)), 1.0)     # rotation keeps RMS
    assert np.allclose(v.reshape(2, -1), x[:, (16 + 1) * 128:(16 + 2) * 128])
    assert np.allclose(q, I.rope(I.rms_norm(x[:, :1024].reshape(2, 8, 128), w, 0.0), [11, 12], 128, 1e4))


# ---------------------------------------------------------------- acceptance rules
from oracle import acceptance as A  # noqa: E402


def test_e4m3_window_rule():
    rng = np.random.default_rng(4)
    x = rng.normal(size=2000) * 30
    b = F.e4m3_encode(x)
    assert A.check_e4m3_within(b, x, 0.0) == (None, 0)
    wrong = b.copy()
    wrong[7] ^= 1                                            # a neighbouring code
    assert A.check_e4m3_within(wrong, x, 0.0)[0] is not None
    # on a midpoint +- a hair, delta admits the other side, and only that
    m = np.float64(F.E4M3_MID[60])
    xs = np.array([m * (1 - 1e-9), m * (1 + 1e-9)])
    other = F.e4m3_encode(xs[::-1])
    assert A.check_e4m3_within(other, xs, 0.0)[0] is not None
    msg, n = A.check_e4m3_within(other, xs, 1e-6 * m)
    assert msg is None and n == 2
    far = F.e4m3_encode(xs * 1.3)
    assert A.check_e4m3_within(far, xs, 1e-6 * m)[0] is not None


def test_nvfp4_window_rule():
    rng = np.random.default_rng(5)
    x = rng.normal(size=(40, 128))
    c, s = N.quantize(x.astype(np.float32))
    assert A.check_nvfp4_within(c, s, x.astype(np.float32).astype(np.float64), 0.0) == (None, 0)
    bad = c.copy()
    bad[3, 10] ^= 0x01                                       # one magnitude step
    assert A.check_nvfp4_within(bad, s, x.astype(np.float32).astype(np.float64), 0.0)[0] is not None
    bad_s = s.copy()
    bad_s[2, 1] += 1
    assert A.check_nvfp4_within(c, bad_s, x.astype(np.float32).astype(np.float64), 0.0)[0] is not None
    # an element on an E2M1 midpoint: the window admits either neighbour
    g = np.zeros((1, 16))
    g[0, 0] = 6.0                                            # amax 6 -> scale 1.0
    g[0, 1] = 1.25 * (1 + 1e-12)                             # just above the 1 | 1.5 midpoint
    cg, sg = N.quantize(g.astype(np.float32))
    assert sg[0, 0] == F.e4m3_encode(1.0)
    alt = cg.copy()
    alt[0, 0] = (alt[0, 0] & 0x0F) | (0x2 << 4)             # magnitude index 2 (1.0) instead of 3
    assert A.check_nvfp4_within(alt, sg, g, 0.0)[0] is not None
    msg, n = A.check_nvfp4_within(alt, sg, g, 1e-6)
    assert msg is None and n == 1
