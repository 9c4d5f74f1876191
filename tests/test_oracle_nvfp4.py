"""Pins of oracle.nvfp4: the pages' byte counts, an exhaustive scale x code
round trip, the dequant-to-FP8 table against torch's float8 cast, and
hand-derived rounding cases."""
import json
import os

import numpy as np
import torch

from oracle import formats as F
from oracle import nvfp4 as N

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")))


def g(k):
    return GOLD[k]["value"]


def test_page_byte_counts():
    heads, d = g("fp8_kv_heads"), g("head_dim")
    fp8_layer = N.kv_bytes_per_token(heads, d, 1, "fp8")
    assert fp8_layer == g("fp8_kv_bytes_per_token_layer")
    # the layer count implied by the FP8 total
    layers = g("kv_bytes_per_token_fp8") // fp8_layer
    assert layers * fp8_layer == g("kv_bytes_per_token_fp8") and layers == 60
    assert N.kv_bytes_per_token(heads, d, layers, "nvfp4") == g("kv_bytes_per_token_nvfp4")
    # the MXFP4 reading (32-element groups) does not give the pages' total
    assert N.kv_bytes_per_token(heads, d, layers, "mxfp4") != g("kv_bytes_per_token_nvfp4")
    saving = 1 - N.kv_bytes_per_token(heads, d, 1, "nvfp4") / fp8_layer
    assert saving == g("kv_saving_fraction")
    # one FP8 index head of dimension 128 is 128 bytes per token per layer
    assert N.fp8_bytes_per_token_head(d) == g("fp8_index_bytes_per_token_layer")
    assert N.nvfp4_bytes_per_token_head(d) == 72


def test_exhaustive_scale_code_round_trip():
    sb = np.arange(1, 127)
    s = F.E4M3_POS[sb]
    rows = []
    want_codes = []
    for code in range(16):
        x = np.zeros((len(sb), 16))
        x[:, 0] = 6.0 * s                       # pins amax / 6 == s exactly
        x[:, 5] = F.E2M1_MAG[code & 7] * s * (-1.0 if code & 8 else 1.0)
        rows.append(x)
        want_codes.append(code)
    x = np.stack(rows).astype(np.float32)      # [16 codes, 126 scales, 16]
    assert np.array_equal(x.astype(np.float64)[..., 0], np.broadcast_to(6.0 * s, x.shape[:2]))
    nib, sc = N.quantize_groups(x)
    assert np.array_equal(sc[..., 0], np.broadcast_to(sb, sc.shape[:2]))
    assert np.all(nib[..., 0] == 7)
    for code in range(16):
        got = nib[code, :, 5]
        want = code if (code & 7) else (code & 8)        # -0 keeps its sign bit
        assert np.all(got == want), (code, got[:5])
    others = np.delete(nib, [0, 5], axis=-1)
    assert np.all(others == 0)


def test_dequant_table_matches_torch_cast():
    sb = np.repeat(np.arange(127, dtype=np.uint8), 16)
    code = np.tile(np.arange(16, dtype=np.uint8), 127)
    # one group per (scale, code); the element sits in slot 0 of the group
    codes = np.zeros((sb.size, 8), dtype=np.uint8)
    codes[:, 0] = code
    fp8, val = N.dequant_fp8(codes, sb[:, None])
    prod = F.E2M1_MAG[code & 7] * F.E4M3_POS[sb] * np.where(code & 8, -1.0, 1.0)
    p32 = prod.astype(np.float32)
    assert np.array_equal(p32.astype(np.float64), prod)                  # exact product
    ref = torch.from_numpy(p32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    inrange = np.abs(prod) < 464
    assert np.array_equal(fp8[inrange, 0], ref[inrange])
    assert np.all(fp8[~inrange, 0] & 0x7F == 0x7E)                        # satfinite
    assert np.array_equal(val[:, 0], F.e4m3_decode(fp8[:, 0]))


def test_scale_rounding_ties_and_neighbours():
    for k in range(125):
        t = 6.0 * F.E4M3_MID[k]
        t32 = np.float32(t)
        assert float(t32) == t                          # exact in fp32
        cases = {t32: k + (k % 2), np.nextafter(t32, np.float32(np.inf)): k + 1,
                 np.nextafter(t32, np.float32(0)): k}
        for amax, want in cases.items():
            x = np.zeros(16, dtype=np.float32)
            x[3] = -amax
            _, sc = N.quantize_groups(x)
            assert sc[0] == want, (k, float(amax), sc[0], want)


def test_element_rounding_hand_cases():
    # s = 1.0 (E4M3 0x38) via amax = 6
    x = np.array([6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0,
                  0.26, 0.74, 1.26, 1.74, 2.6, 3.4, 4.9, -0.01], dtype=np.float32)
    nib, sc = N.quantize_groups(x)
    assert sc[0] == 0x38
    assert nib.tolist() == [7, 0, 2, 2, 4, 4, 6, 6, 1, 1, 3, 3, 5, 5, 6, 8]


def test_saturation_and_zero_scale():
    x = np.zeros(16, dtype=np.float32)
    x[0], x[1] = 3000.0, -2900.0
    nib, sc = N.quantize_groups(x)
    assert sc[0] == 0x7E and nib[0] == 7 and nib[1] == 15
    tiny = np.full(16, -(6.0 * 2.0 ** -10), dtype=np.float32)
    nib, sc = N.quantize_groups(tiny)
    assert sc[0] == 0 and np.all(nib == 8)
    z = np.zeros(16, dtype=np.float32)
    nib, sc = N.quantize_groups(z)
    assert sc[0] == 0 and np.all(nib == 0)


def test_pack_unpack_order():
    nib = np.arange(16, dtype=np.uint8)
    packed = N.pack_nibbles(nib)
    assert packed.tolist() == [0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE]
    assert np.array_equal(N.unpack_nibbles(packed), nib)


def test_quantization_error_bounded_by_half_step():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((64, 4, 128)).astype(np.float32)
    c, s = N.quantize(x)
    nib = N.unpack_nibbles(c)
    sv = F.e4m3_decode(np.repeat(s, 16, axis=-1))
    recon = F.E2M1_MAG[nib & 7] * sv * np.where(nib & 8, -1, 1)
    # nearest rounding: error at most half the gap to the neighbouring E2M1 value
    # (gaps 0.5, 0.5, 0.5, 0.5, 1, 1, 2) unless clipped at 6*s
    r = np.abs(x) / sv
    err = np.abs(recon - x) / sv
    bound = np.where(r <= 2, 0.25, np.where(r <= 4, 0.5, 1.0))
    clipped = r > 6
    assert np.all(err[~clipped] <= bound[~clipped] + 1e-12)


def test_pool_write_and_gather_round_trip():
    rng = np.random.default_rng(9)
    src = rng.standard_normal((300, 2, 128)).astype(np.float32)
    codes, scales = N.empty_pool(5, 2, fill=0xAB)
    slots = np.array([(7 * t) % 640 for t in range(300)])
    slots[10] = -1
    N.write_cache(codes, scales, src, slots)
    c, s = N.quantize(src)
    for t in (0, 1, 127, 299):
        sl = slots[t]
        assert np.array_equal(codes[sl // 128, :, sl % 128], c[t])
        assert np.array_equal(scales[sl // 128, :, sl % 128], s[t])
    assert np.all(codes[(7 * 10) // 128, :, (7 * 10) % 128] == 0xAB)   # skipped slot untouched
    bt = np.array([3, 0, 4])
    gc, gs = N.gather_sequence(codes, scales, bt, 300)
    assert gc.shape == (300, 2, 64)
    assert np.array_equal(gc[130], codes[0, :, 2]) and np.array_equal(gs[299], scales[4, :, 43])
